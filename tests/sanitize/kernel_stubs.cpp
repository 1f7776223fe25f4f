// Host-only stand-ins for the kernel launchers of libstc, so that the host
// code (validation, eigensolver, water-filling, Lloyd, state building) can be
// built with the address and undefined-behaviour sanitizers and exercised
// without a GPU. Every launcher reports failure; the sanitized driver only
// runs paths that return before any launch.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../spectral_transform_codec_amd/csrc/stc_internal.h"

namespace stc {
int launch_gram(const void*, int, int64_t, int64_t, int64_t, int64_t, double*, int64_t, void*) { return 1; }
int launch_encode_eigen(const EncodeLaunch&, void*) { return 1; }
int launch_sketch_eigen(const EncodeLaunch&, void*) { return 1; }
int launch_decode_eigen(const DecodeLaunch&, void*) { return 1; }
int launch_encode_rht(const EncodeLaunch&, void*) { return 1; }
int launch_decode_rht(const DecodeLaunch&, void*) { return 1; }
int launch_attend(const AttendLaunch&, void*) { return 1; }
size_t attend_scratch_bytes() { return 0; }
int attend_scratch(void**) { return 1; }
int read_debug_flags(unsigned* out, void*) {
  *out = 0u;
  return 0;
}
int debug_build() { return 0; }
int launch_stream_copy(void*, const void*, int64_t, void*) { return 1; }
}  // namespace stc
