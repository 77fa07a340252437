// Host-side driver of libcsa's validation layer (no GPU needed): every case returns before a
// launch. It checks the status codes of invalid and edge-case calls and times the full host
// validation and workspace carving of csa_decode_step per call.
//
// "DeepSeek V4-Flash: The Cost of Deciding What to Read", section "TileLang, and a theorem
// prover in the compiler": contract checks on the host belong in compiled code and cost under a
// microsecond per call.
//
// Usage: abi_host_driver [timing_calls]   (prints "ok" and "validate_ns_per_call <x>")
#include <chrono>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "csa.h"

namespace {

int failures = 0;

void expect(const char* what, int got, int want) {
  if (got != want) {
    std::printf("FAIL %s: status %d, expected %d\n", what, got, want);
    ++failures;
  }
}

void* const kFake = reinterpret_cast<void*>(static_cast<uintptr_t>(256));   // never dereferenced

csa_decode_desc base_desc() {
  csa_decode_desc d;
  std::memset(&d, 0, sizeof(d));
  d.dtype = CSA_BF16;
  d.m = 4; d.dim = 512; d.n_heads = 64; d.idx_heads = 64; d.idx_dim = 128;
  d.top_k = 512; d.window = 128; d.w_cap = 128; d.n_attn = 1;
  d.n_seq = 4; d.e_cap = 262144; d.scale = 0.0442f;
  return d;
}

// every pointer a step needs, set to a fake address
csa_decode_desc full_desc() {
  csa_decode_desc d = base_desc();
  const void** cp[] = {(const void**)&d.pos, &d.x_new, &d.z_new, &d.xi_new, &d.zi_new, &d.bias,
                       &d.bias_i, &d.q_idx, (const void**)&d.w};
  for (auto p : cp) *p = kFake;
  void** mp[] = {&d.kv, &d.k_idx, &d.x_tail, &d.z_tail, &d.xi_tail, &d.zi_tail};
  for (auto p : mp) *p = kFake;
  d.out_idx = static_cast<int32_t*>(kFake);
  d.q[0] = kFake; d.win[0] = kFake; d.win_new[0] = kFake; d.out[0] = kFake;
  d.sink[0] = static_cast<const float*>(kFake);
  return d;
}

}  // namespace

int main(int argc, char** argv) {
  const long calls = argc > 1 ? std::atol(argv[1]) : 200000;
  expect("abi version", csa_abi_version(), CSA_ABI_VERSION);
  for (int st = -7; st <= 0; ++st)
    if (csa_status_str(st) == nullptr || std::strlen(csa_status_str(st)) == 0) ++failures;

  // compress / c4a / norm_rope / quantisers: nulls, shapes, dtypes
  expect("compress null", csa_compress(nullptr, kFake, kFake, kFake, 1, 8, 0, 64, 4, CSA_BF16, nullptr), CSA_ERR_NULL);
  expect("compress n_tok % m", csa_compress(kFake, kFake, kFake, kFake, 1, 7, 0, 64, 4, CSA_BF16, nullptr), CSA_ERR_SHAPE);
  expect("compress dtype", csa_compress(kFake, kFake, kFake, kFake, 1, 8, 0, 64, 4, 7, nullptr), CSA_ERR_DTYPE);
  expect("compress m", csa_compress(kFake, kFake, kFake, kFake, 1, 1024, 0, 64, 129, CSA_BF16, nullptr), CSA_ERR_SHAPE);
  expect("compress empty", csa_compress(kFake, kFake, kFake, kFake, 0, 8, 0, 64, 4, CSA_BF16, nullptr), CSA_OK);
  expect("c4a one prev", csa_compress_c4a(kFake, kFake, kFake, kFake, kFake, kFake, kFake, nullptr, kFake, 1, 8, 0, 64, 4, CSA_BF16, nullptr), CSA_ERR_NULL);
  expect("norm_rope flags", csa_norm_rope(kFake, nullptr, nullptr, kFake, 1, 1, 64, 0, 10000.f, 1e-6f, 8, CSA_BF16, nullptr), CSA_ERR_SHAPE);
  expect("mxfp4 dim", csa_quantize_mxfp4(kFake, kFake, kFake, 1, 48, CSA_BF16, nullptr), CSA_ERR_SHAPE);
  void* const kOdd = reinterpret_cast<void*>(static_cast<uintptr_t>(256 + 8));   // not 16-aligned
  expect("kv_fp8 align", csa_quantize_kv_fp8(kFake, kOdd, 1, CSA_BF16, nullptr), CSA_ERR_SHAPE);
  expect("kv_fp4 align", csa_quantize_kv_fp4(kFake, kOdd, 1, CSA_BF16, nullptr), CSA_ERR_SHAPE);
  expect("kv_fp4 null", csa_dequantize_kv_fp4(nullptr, kFake, 1, nullptr), CSA_ERR_NULL);
  expect("kv_fp4 empty", csa_dequantize_kv_fp4(kFake, kFake, 0, nullptr), CSA_OK);

  // index / attention
  const size_t iws = csa_index_topk_workspace_size(4, 1, 262144, 512);
  if (iws == 0 || iws % 256 != 0) ++failures;
  expect("index_topk no ws", csa_index_topk(kFake, (const float*)kFake, kFake, (const int64_t*)kFake, nullptr, nullptr, 0, 4, 1, 262144, 64, 128, 4, 512, (int32_t*)kFake, nullptr, nullptr, nullptr, 0, CSA_BF16, nullptr), CSA_ERR_WORKSPACE);
  expect("index_topk top_k", csa_index_topk(kFake, (const float*)kFake, kFake, (const int64_t*)kFake, nullptr, nullptr, 0, 4, 1, 262144, 64, 128, 4, 4096, (int32_t*)kFake, nullptr, nullptr, kFake, iws, CSA_BF16, nullptr), CSA_ERR_SHAPE);
  expect("sparse_attn heads", csa_sparse_attn(kFake, kFake, (const int32_t*)kFake, 512, kFake, 128, 128, (const int64_t*)kFake, nullptr, 0.04f, kFake, 4, 1, 1024, 65, 512, kFake, 1 << 30, CSA_BF16, nullptr), CSA_ERR_SHAPE);
  expect("sparse_attn_fp4 dtype", csa_sparse_attn_fp4(kFake, kFake, (const int32_t*)kFake, 512, kFake, 128, 128, (const int64_t*)kFake, nullptr, 0.04f, kFake, 4, 1, 1024, 64, 512, kFake, 1 << 30, CSA_F32, nullptr), CSA_ERR_UNSUPPORTED);
  expect("sparse_attn window", csa_sparse_attn(kFake, kFake, (const int32_t*)kFake, 512, kFake, 64, 128, (const int64_t*)kFake, nullptr, 0.04f, kFake, 4, 1, 1024, 64, 512, kFake, 1 << 30, CSA_BF16, nullptr), CSA_ERR_SHAPE);

  // decode step
  csa_decode_desc d = full_desc();
  const size_t need = csa_decode_step_workspace_size(&d);
  if (need == 0 || need % 256 != 0) ++failures;
  expect("decode null desc", csa_decode_step(nullptr, nullptr, 0, nullptr), CSA_ERR_NULL);
  expect("decode small ws", csa_decode_step(&d, kFake, need - 1, nullptr), CSA_ERR_WORKSPACE);
  csa_decode_desc e = d; e.n_attn = CSA_MAX_ATTN + 1;
  expect("decode n_attn", csa_decode_step(&e, kFake, need, nullptr), CSA_ERR_SHAPE);
  e = d; e.out[0] = nullptr;
  expect("decode out null", csa_decode_step(&e, kFake, need, nullptr), CSA_ERR_NULL);
  e = d; e.scan_events[0] = kFake;
  expect("decode one scan event", csa_decode_step(&e, kFake, need, nullptr), CSA_ERR_NULL);
  e = d; e.block_size = 64; e.max_blocks = 1024; e.q_idx2 = kFake; e.w2 = (const float*)kFake;
  expect("decode pool too big", csa_decode_step(&e, kFake, need, nullptr), CSA_ERR_UNSUPPORTED);
  e = d; e.kv_format = CSA_KV_FP4; e.kv = kOdd;
  expect("decode fp4 align", csa_decode_step(&e, kFake, need, nullptr), CSA_ERR_SHAPE);
  e = d; e.kv_rope_dim = 3;
  expect("decode odd rope", csa_decode_step(&e, kFake, need, nullptr), CSA_ERR_SHAPE);
  e = d; e.idx_format = CSA_IDX_MXFP4;   // codes need their scale bytes
  expect("decode mxfp4 scales", csa_decode_step(&e, kFake, need, nullptr), CSA_ERR_NULL);
  e = d; e.n_seq = 64;                   // 64 x 1M entries: beyond the static scratch
  expect("noalloc beyond scratch", csa_decode_step_noalloc(&e, nullptr), CSA_ERR_WORKSPACE);
  expect("noalloc null", csa_decode_step_noalloc(nullptr, nullptr), CSA_ERR_NULL);

  // timing: the full validation and workspace carving of a valid descriptor, refused only by
  // the workspace size check that follows them (nothing is launched)
  volatile int sink = 0;
  const auto t0 = std::chrono::steady_clock::now();
  for (long i = 0; i < calls; ++i) sink += csa_decode_step(&d, kFake, need - 1, nullptr);
  const auto t1 = std::chrono::steady_clock::now();
  const double ns = std::chrono::duration<double, std::nano>(t1 - t0).count() / double(calls);
  if (sink != -5 * calls) ++failures;
  std::printf("validate_ns_per_call %.1f\n", ns);
  if (failures) {
    std::printf("%d failures\n", failures);
    return 1;
  }
  std::printf("ok\n");
  return 0;
}
