// Host-only stand-ins for the kernel launchers of libfa, so that the C ABI's
// argument validation and parameter set-up (fa_api.cpp) can be built and run
// under AddressSanitizer and UndefinedBehaviorSanitizer on a machine without a
// GPU. Each stub checks the invariants its real launcher relies on (positive
// sizes, a grid below 2^31 workgroups, the pointers the kernels dereference)
// and counts the call; nothing is dereferenced. The two HIP runtime queries
// fa_api.cpp makes report that no device is present.
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "fa_noalloc.h"
#include "fa_params.h"

namespace {
long long g_launches = 0;
constexpr int64_t kMaxGrid = (int64_t(1) << 31) - 1;

void require(bool ok, const char* what) {
  if (!ok) {
    fprintf(stderr, "launcher invariant violated: %s\n", what);
    abort();
  }
}

void check_fwd(const fa::FwdParams& p, int64_t groups) {
  require(p.B > 0 && p.H > 0 && p.Nq > 0 && p.Nk >= 0, "forward sizes");
  require(groups > 0 && groups <= kMaxGrid, "forward grid");
  require(p.scale_log2 > 0.0f, "forward scale");
  ++g_launches;
}
}  // namespace

extern "C" long long fa_stub_launches() { return g_launches; }

extern "C" hipError_t hipGetDevice(int*) { return hipErrorNoDevice; }
extern "C" hipError_t hipDeviceGetAttribute(int*, hipDeviceAttribute_t, int) {
  return hipErrorNoDevice;
}

namespace fa {

template <int D, bool SOFTCAP, bool ALIBI, int MODE>
int launch_fwd_bf16(const FwdParams& p, void*) {
  const int64_t splits = MODE != FWD_CONTIG ? p.num_splits : 1;
  require(p.q && (p.k || p.total_k == 0) && (p.v || p.total_k == 0), "forward inputs");
  require(MODE == FWD_CONTIG ? p.o != nullptr : (p.o_part && p.lse_part), "forward outputs");
  require(MODE < FWD_PAGED_SPLIT || p.block_table, "block table");
  // Page tiles: every wavefront's 16-row slab of a 64-key tile inside one page.
  require(MODE != FWD_PAGED_TILES || (p.page_size % 16 == 0 && !p.k_new), "bf16 page tiles");
  require(p.appended == 0 || (MODE == FWD_PAGED_TILES && p.seqlens_k && p.Nk >= p.appended),
          "pass after an append");
  check_fwd(p, (int64_t)p.num_q_tiles * p.H * p.B * splits);
  return 0;
}
template <int D, bool SOFTCAP, bool ALIBI, bool PAGED>
int launch_fwd_f32(const FwdParams& p, void*) {
  require(p.q && (p.o || (p.o_part && p.lse_part)), "fp32 forward pointers");
  check_fwd(p, (int64_t)p.num_q_tiles * p.H * p.B * (PAGED ? p.num_splits : 1));
  return 0;
}
template <int D, bool SOFTCAP, bool ALIBI, int MODE>
int launch_fwd_fp8(const FwdParams& p, void*) {
  constexpr bool SPLIT = MODE != FWD_CONTIG;

  require(p.q && p.k && p.v && (SPLIT ? (p.o_part && p.lse_part) : p.o != nullptr),
          "fp8 forward pointers");
  require(MODE != FWD_CONTIG_SPLIT || (p.num_splits >= 1 && p.split_align == 128),
          "fp8 split chunking");
  // Paged: chunks of whole pages, a table that covers every key; page tiles
  // need every wavefront's 32-row slab of a 128-key tile inside one page.
  require(MODE < FWD_PAGED_SPLIT ||
              (p.block_table && p.page_size > 0 && p.split_align == p.page_size &&
               p.max_pages > 0 && (int64_t)p.max_pages * p.page_size >= p.Nk &&
               (p.page_shift < 0 || (1 << p.page_shift) == p.page_size)),
          "fp8 paged cache");
  require(MODE != FWD_PAGED_TILES || p.page_size % 32 == 0, "fp8 page tiles");
  check_fwd(p, (int64_t)p.num_q_tiles * p.H * p.B * (SPLIT ? p.num_splits : 1));
  return 0;
}
template <int D, bool SOFTCAP, bool ALIBI, bool APPEND>
int launch_decode_bf16(const FwdParams& p, void*) {
  require(p.q && p.k && p.v && p.block_table && p.o_part && p.lse_part, "decode pointers");
  require(!APPEND || (p.k_new && p.v_new), "append rows");
  check_fwd(p, (int64_t)p.H * p.B * p.num_splits);
  return 0;
}
template <int D>
int launch_append_bf16(const FwdParams& p, void*) {
  require(p.k_new && p.v_new && p.k && p.v && p.block_table && p.seqlens_k, "append pointers");
  require(p.Nq >= 1 && p.Nk >= p.Nq && p.appended == 0, "append sizes");
  ++g_launches;
  return 0;
}
template <int D, bool SOFTCAP, bool ALIBI>
int launch_decode_fp8(const FwdParams& p, void*) {
  require(p.q && p.k && p.v && p.block_table && p.o_part && p.lse_part, "fp8 decode pointers");
  check_fwd(p, (int64_t)p.H * p.B * p.num_splits);
  return 0;
}
template <int D>
int launch_combine(const CombineParams& p, void*) {
  require(p.o_part && p.lse_part && p.o, "combine pointers");
  require(p.S > 0 && p.B > 0 && p.H > 0 && p.Nq > 0, "combine sizes");
  require(((int64_t)p.B * p.H * p.Nq + 3) / 4 <= kMaxGrid, "combine grid");
  ++g_launches;
  return 0;
}
template <int D, bool SOFTCAP, bool ALIBI>
int launch_bwd_bf16(const BwdParams& p, void*) {
  require(p.rowterms != nullptr, "row-term workspace");
  require(p.B > 0 && p.H > 0 && p.Nq > 0 && p.Nk > 0 && p.nblk > 0, "backward sizes");
  require((int64_t)p.num_q_tiles * p.H * p.B <= kMaxGrid &&
              (int64_t)p.num_k_tiles * p.H * p.B <= kMaxGrid,
          "backward grid");
  ++g_launches;
  return 0;
}

// fa_bwd_noalloc's buffer: a host array stands in for the device one (never
// dereferenced by the stubs).
int noalloc_scratch(float** out) {
  static float host_stand_in[16];
  *out = host_stand_in;
  return 0;
}

#define STUB_D(D)                                                                      \
  template int launch_combine<D>(const CombineParams&, void*);                        \
  template int launch_append_bf16<D>(const FwdParams&, void*);                        \
  STUB_SA(D, false, false) STUB_SA(D, false, true) STUB_SA(D, true, false) STUB_SA(D, true, true)
#define STUB_SA(D, SC, AL)                                                             \
  template int launch_fwd_bf16<D, SC, AL, 0>(const FwdParams&, void*);                \
  template int launch_fwd_bf16<D, SC, AL, 1>(const FwdParams&, void*);                \
  template int launch_fwd_bf16<D, SC, AL, 2>(const FwdParams&, void*);                \
  template int launch_fwd_bf16<D, SC, AL, 3>(const FwdParams&, void*);                \
  template int launch_fwd_f32<D, SC, AL, false>(const FwdParams&, void*);             \
  template int launch_fwd_f32<D, SC, AL, true>(const FwdParams&, void*);              \
  template int launch_decode_bf16<D, SC, AL, false>(const FwdParams&, void*);         \
  template int launch_decode_bf16<D, SC, AL, true>(const FwdParams&, void*);          \
  template int launch_decode_fp8<D, SC, AL>(const FwdParams&, void*);                 \
  template int launch_fwd_fp8<D, SC, AL, FWD_CONTIG>(const FwdParams&, void*);        \
  template int launch_fwd_fp8<D, SC, AL, FWD_CONTIG_SPLIT>(const FwdParams&, void*);  \
  template int launch_fwd_fp8<D, SC, AL, FWD_PAGED_TILES>(const FwdParams&, void*);   \
  template int launch_fwd_fp8<D, SC, AL, FWD_PAGED_SPLIT>(const FwdParams&, void*);   \
  template int launch_bwd_bf16<D, SC, AL>(const BwdParams&, void*);
STUB_D(64)
STUB_D(128)

}  // namespace fa
