// The static row-term buffer of fa_bwd_noalloc (defined in fa_bwd_bf16.hip).
#pragma once

namespace fa {

constexpr long long NOALLOC_SCRATCH_BYTES = 16LL << 20;  // FA_NOALLOC_SCRATCH_BYTES in fa.h
constexpr long long NOALLOC_SCRATCH_FLOATS = NOALLOC_SCRATCH_BYTES / 4;

// Device address of the buffer on the current device (looked up once per
// device and kept); returns a hipError_t as int.
int noalloc_scratch(float** out);

}  // namespace fa
