// Paged causal extend attention (MFMA). Filled in below.
#pragma once
#include "common.hpp"
