// Batched sampler kernels. Filled in below.
#pragma once
#include "common.hpp"
