"""Request length arithmetic (oracle side; test infrastructure only).

Follows "核心数据结构：Req、Batch、Context", section "Req：请求的三个长度":
a request's state is three lengths -- cached_len (tokens whose KV is already
in the pool), device_len (tokens whose KV will be in the pool after this
forward) and max_device_len = prompt length + max_tokens. Everything the
kernels need is derived from them: extend_len = device_len - cached_len is
the number of query rows this step, and the attention of this step sees
device_len keys. complete_one() moves every computed token into the cache and
asks for one more position next step.
"""


class Req:
    def __init__(self, prompt_len: int, cached_len: int, output_len: int):
        self.cached_len = int(cached_len)
        self.device_len = int(prompt_len)
        self.max_device_len = int(prompt_len) + int(output_len)
        if not (0 <= self.cached_len < self.device_len <= self.max_device_len):
            raise ValueError("need 0 <= cached_len < device_len <= max_device_len")

    @property
    def extend_len(self) -> int:
        return self.device_len - self.cached_len

    @property
    def remain_len(self) -> int:
        return self.max_device_len - self.device_len

    @property
    def can_decode(self) -> bool:
        return self.remain_len > 0

    def complete_one(self) -> None:
        self.cached_len = self.device_len
        self.device_len += 1

    def lengths(self):
        """(cached_len, device_len, extend_len, remain_len)."""
        return (self.cached_len, self.device_len, self.extend_len, self.remain_len)
