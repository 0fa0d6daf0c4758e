// Sanitizer check program for the host side of libmla_decode
// (sparse_mla_amd/csrc/mla_api.cpp): built by tests/test_sanitizers.py with
// AddressSanitizer and UndefinedBehaviorSanitizer against stub launchers that
// record the kernel arguments instead of launching (no GPU, no HIP).  It
// drives every entry point with valid and invalid arguments, including the
// extreme sizes the checks guard (65536 rows, 64 splits, 2 GiB spans), and
// checks the statuses and the arguments that reach the launchers.
#include <stdint.h>
#include <stdio.h>

#include <initializer_list>

#include "mla_decode.h"
#include "mla_kernels.h"

namespace mla {
static int n_launch = 0;
static DecodeArgs last_decode;
static AbsorbArgs last_absorb;
static ValueUpArgs last_vu;
static CombineArgs last_combine;
static OutProjArgs last_oproj;
int launch_absorb(const AbsorbArgs& a, void*) { last_absorb = a; ++n_launch; return 0; }
int launch_decode(const DecodeArgs& a, void*) { last_decode = a; ++n_launch; return 0; }
int launch_combine(const CombineArgs& a, void*) { last_combine = a; ++n_launch; return 0; }
int launch_value_up(const ValueUpArgs& a, void*) { last_vu = a; ++n_launch; return 0; }
int launch_dequant(const DequantArgs&, void*) { ++n_launch; return 0; }
int launch_output_proj(const OutProjArgs& a, void*) { last_oproj = a; ++n_launch; return 0; }
int launch_output_proj_pack(const uint16_t*, uint16_t*, void*) { ++n_launch; return 0; }
int launch_output_proj_split(const OutProjArgs& a, void*) { last_oproj = a; ++n_launch; return 0; }
int device_cu_count(int* cus) { *cus = 256; return 0; }
static char fake_scratch[256] __attribute__((aligned(256)));
int scratch_buffer(void** ptr) { *ptr = fake_scratch; return 0; }
}  // namespace mla

#define CHECK(c)                                                    \
  do {                                                              \
    if (!(c)) {                                                     \
      fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
      return 1;                                                     \
    }                                                               \
  } while (0)

static void* P(uintptr_t a) { return reinterpret_cast<void*>(a); }

int main() {
  const uintptr_t F = 1u << 20;  // a 16-byte aligned address, never dereferenced
  int32_t S = 0;
  for (int32_t B : {1, 7, 32, 64, 128, 65536})
    for (int32_t k : {1, 33, 1001, 2048, 8192, 131072}) {
      for (int dense = 0; dense < 2; ++dense) {
        const int st = mla_plan(B, k, dense, 256, &S);
        if (!dense && k > 64 * 1024) { CHECK(st == MLA_ERR_BAD_DIM || (st == MLA_OK && S >= 1)); continue; }
        CHECK(st == MLA_OK && S >= 1 && S <= MLA_MAX_SPLITS);
      }
    }
  CHECK(mla_workspace_bytes(65536, 64) == (size_t)64 * 65536 * 128 * (1024 + 8));
  // A valid sparse decode reaches the launcher with the documented split chunk.
  const size_t ws = mla_workspace_bytes(64, 4);
  int st = mla_sparse_decode(P(F), P(F), 8192, 64, P(F), 576 * 32768, 576, P(F + 1024), 576 * 32768, 576, (const int32_t*)P(F),
                             32768, (const int32_t*)P(F), 2048, 0.07f, 64, 4, P(F), ws, P(F), (float*)P(F), 0, nullptr, 0,
                             nullptr, nullptr, nullptr);
  CHECK(st == MLA_OK && mla::last_decode.chunk == 512 && mla::last_decode.H == 128 && mla::last_decode.causal == 0);
  CHECK((char*)mla::last_decode.part_ml == (char*)P(F) + (size_t)4 * 64 * 128 * 1024);
  // Extreme sizes: spans just past 2 GiB are refused.
  st = mla_sparse_decode(P(F), P(F), 8192, 64, P(F), 0, 576, P(F), 0, 576, (const int32_t*)P(F), 1864136,
                         (const int32_t*)P(F), 64, 0.07f, 1, 1, nullptr, 0, P(F), nullptr, 0, nullptr, 0, nullptr, nullptr,
                         nullptr);
  CHECK(st == MLA_ERR_RANGE);
  st = mla_sparse_decode(P(F), P(F), 8192, 64, P(F), 0, 576, P(F), 0, 576, (const int32_t*)P(F), 100, (const int32_t*)P(F),
                         64, 0.07f, 65537, 1, nullptr, 0, P(F), nullptr, 0, nullptr, 0, nullptr, nullptr, nullptr);
  CHECK(st == MLA_ERR_BAD_DIM);
  // Head-sharded calls.
  for (int32_t H : {16, 32, 64}) {
    const size_t wsh = mla_workspace_bytes_heads(H, 64, 4);
    st = mla_sparse_decode_heads(H, P(F), P(F), H * 64, 64, P(F), 576 * 4096, 576, P(F + 1024), 576 * 4096, 576,
                                 (const int32_t*)P(F), 4096, (const int32_t*)P(F), 2048, 0.07f, 64, 4, P(F), wsh, P(F),
                                 nullptr, 0, nullptr, 0, nullptr, nullptr, nullptr);
    CHECK(st == MLA_OK && mla::last_decode.H == H);
    CHECK(mla_combine_value_up_heads(H, P(F), wsh, 64, 4, P(F), P(F), H * 128, 128, nullptr, nullptr, nullptr) == MLA_OK);
    CHECK(mla::last_vu.H == H && mla::last_vu.S == 4);
    CHECK(mla_combine_heads(H, P(F), wsh, 64, 4, P(F), nullptr, nullptr, nullptr) == MLA_OK && mla::last_combine.H == H);
    CHECK(mla_absorb_q_heads(H, P(F), H * 128, 128, P(F), P(F), 64, nullptr) == MLA_OK && mla::last_absorb.H == H);
  }
  CHECK(mla_absorb_q_heads(48, P(F), 8192, 128, P(F), P(F), 64, nullptr) == MLA_ERR_UNSUPPORTED);
  // Allocation-free decode: the partials land in the static scratch.
  const int before = mla::n_launch;
  st = mla_sparse_decode_noalloc(P(F), P(F), 8192, 64, P(F), 576 * 4096, 576, P(F + 1024), 576 * 4096, 576,
                                 (const int32_t*)P(F), 4096, (const int32_t*)P(F), 2048, 0.07f, 64, 4, P(F), nullptr, 0,
                                 nullptr, 0, nullptr, nullptr, nullptr);
  CHECK(st == MLA_OK && mla::n_launch == before + 2 && (char*)mla::last_combine.part_o == mla::fake_scratch);
  CHECK(mla_sparse_decode_noalloc(P(F), P(F), 8192, 64, P(F), 0, 576, P(F), 0, 576, (const int32_t*)P(F), 2048,
                                  (const int32_t*)P(F), 2048, 0.07f, 128, 64, P(F), nullptr, 0, nullptr, 0, nullptr, nullptr,
                                  nullptr) == MLA_ERR_SCRATCH_LIMIT);
  // Prefill: B*T rows, causal rows, workspace split into q_abs and partials.
  const size_t pws = mla_prefill_workspace_bytes(1, 4096, 2);
  st = mla_sparse_prefill(P(F), 16384, 128, P(F), 8192, 64, P(F), 0, 576, P(F + 1024), 0, 576, P(F),
                          (const int32_t*)P(F), 2048, 0.07f, 1, 4096, 2, P(F), pws, P(F), 16384, 128, nullptr, 0, nullptr,
                          0, nullptr, nullptr);
  CHECK(st == MLA_OK && mla::last_decode.causal == 1 && mla::last_decode.rows_per_seq == 4096 &&
        mla::last_decode.B == 4096 && mla::last_absorb.B == 4096 && mla::last_vu.B == 4096);
  CHECK(mla_prefill_workspace_bytes(65536, 2, 2) == 0);
  CHECK(mla_sparse_prefill(P(F), 16384, 128, P(F), 8192, 64, P(F), 0, 576, P(F + 1024), 0, 576, P(F),
                           (const int32_t*)P(F), 2048, 0.07f, 1, 4096, 2, P(F), pws, P(F), 16384, 128, nullptr,
                           MLA_FLAG_WRITE_SCORES, nullptr, 0, nullptr, nullptr) == MLA_ERR_BAD_DIM);
  // fp8 weights.
  CHECK(mla_absorb_q_fp8(P(F), 16384, 128, P(F), (const float*)P(F), P(F), 64, nullptr, nullptr) == MLA_OK);
  CHECK(mla::last_absorb.fp8.w_fp8 != nullptr && mla::last_absorb.wkv_b == nullptr);
  CHECK(mla_value_up_fp8(P(F), P(F), (const float*)P(F + 2), P(F), 16384, 128, 4, nullptr, nullptr) == MLA_ERR_ALIGNMENT);
  // Output projection: one launch per 64 rows.
  const int b0 = mla::n_launch;
  CHECK(mla_output_proj(P(F), 16384, P(F), P(F), 7168, 100, nullptr) == MLA_OK && mla::n_launch == b0 + 2);
  CHECK(mla::last_oproj.B == 36);
  CHECK(mla_output_proj(P(F), (int64_t)1 << 26, P(F), P(F), 7168, 4, nullptr) == MLA_ERR_RANGE);
  CHECK(!mla::last_oproj.packed);
  CHECK(mla_output_proj_packed(P(F), 16384, P(F), P(F), 7168, 70, nullptr) == MLA_OK && mla::last_oproj.packed &&
        mla::last_oproj.B == 6);
  CHECK(mla_output_proj_pack(P(F), P(F + 16), nullptr) == MLA_OK);
  CHECK(mla_output_proj_pack(P(F), P(F + 2), nullptr) == MLA_ERR_ALIGNMENT);
  // Split over the inputs: a workspace of 4 x min(B, 64) x 7168 floats, one launch per 64 rows.
  CHECK(mla_output_proj_split_workspace_bytes(1) == 4u * 7168u * 4u);
  CHECK(mla_output_proj_split_workspace_bytes(100) == 4u * 64u * 7168u * 4u);
  CHECK(mla_output_proj_split_workspace_bytes(0) == 0 && mla_output_proj_split_workspace_bytes(65537) == 0);
  {
    const size_t need = mla_output_proj_split_workspace_bytes(100);
    const int b1 = mla::n_launch;
    CHECK(mla_output_proj_split(P(F), 16384, P(F), P(F), 7168, 100, P(F), need, nullptr) == MLA_OK &&
          mla::n_launch == b1 + 2 && mla::last_oproj.B == 36 && mla::last_oproj.part == P(F) &&
          !mla::last_oproj.packed);
    CHECK(mla_output_proj_split(P(F), 16384, P(F), P(F), 7168, 100, P(F), need - 1, nullptr) ==
          MLA_ERR_WORKSPACE_TOO_SMALL);
    CHECK(mla_output_proj_split(P(F), 16384, P(F), P(F), 7168, 100, nullptr, need, nullptr) == MLA_ERR_NULL_POINTER);
    CHECK(mla_output_proj_split(P(F), 16384, P(F), P(F), 7168, 100, P(F + 4), need, nullptr) == MLA_ERR_ALIGNMENT);
    CHECK(mla_output_proj_split(P(F), 16384, P(F), P(F), 7168, 0, P(F), need, nullptr) == MLA_ERR_BAD_DIM);
    CHECK(mla_output_proj(P(F), 16384, P(F), P(F), 7168, 3, nullptr) == MLA_OK && mla::last_oproj.part == nullptr);
  }
  for (int code = 0; code <= 8; ++code) CHECK(mla_status_string(code) != nullptr);
  puts("api sanitizer check: ok");
  return 0;
}
