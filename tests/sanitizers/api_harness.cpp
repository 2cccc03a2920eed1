// Host-only harness for the C ABI's argument checks, built with
// AddressSanitizer and UndefinedBehaviorSanitizer (no GPU code).
//
// sas_api.cpp is linked against stand-ins for the kernel launchers and for
// the few HIP runtime calls it makes, so every entry point runs its checks
// with good and bad arguments and "launches" nothing.  Host arrays are
// allocated at exactly their documented sizes, so a check that reads past
// one is reported by the sanitizer.  Exit status 0 = every expectation met.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstring>
#include <vector>

#include "sas.h"
#include "sas_launch.h"

static int g_launches = 0;
static int g_failures = 0;

namespace sas {
hipError_t launch_gate_topk(const GateParams &, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_gate_bwd(const GateBwdParams &, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_fwd(const FwdParams &, int, int, int, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_bwd_prepare(const BwdParams &, hipStream_t) { ++g_launches; return hipSuccess; }
bool bwd_dq_supported(const BwdParams &p, int, int) { return p.Kb <= 100; }
hipError_t launch_bwd_dq(const BwdParams &, int, int, int, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_bwd_dkdv(const BwdParams &, int, int, int, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_pool_keys(const DecodeParams &, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_decode_append(const DecodeParams &, const void *, const void *, void *, void *,
                                hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_decode_select(const DecodeParams &, const SelectParams &, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_decode_attend(const DecodeParams &, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_decode_select_fine(const DecodeParams &, const HierParams &, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_pool_coarse(const DecodeParams &, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
static float g_scratch_standin[16];
hipError_t decode_scratch_address(float **out) {
  *out = g_scratch_standin;
  return hipSuccess;
}
}  // namespace sas

// HIP runtime stand-ins (the runtime itself is not linked).
hipError_t hipGetDevice(int *d) {
  *d = 0;
  return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int *v, hipDeviceAttribute_t, int) {
  *v = 256;
  return hipSuccess;
}
hipError_t hipGetLastError(void) { return hipSuccess; }
const char *hipGetErrorString(hipError_t) { return "stand-in"; }

static void expect(const char *what, sas_status got, sas_status want) {
  if (got != want) {
    std::printf("FAIL %s: status %d, expected %d (%s)\n", what, got, want, sas_last_error());
    ++g_failures;
  }
}

static void *const D = reinterpret_cast<void *>(0x10000);  // stand-in device pointer
static float *const DF = reinterpret_cast<float *>(0x10000);
static int32_t *const DI = reinterpret_cast<int32_t *>(0x10000);

int main() {
  // -------------------------------------------------- varlen problems
  const int nseq = 2;
  int32_t *cu = new int32_t[nseq + 1]{0, 200, 264};
  int32_t *cuq = new int32_t[nseq + 1]{0, 4, 5};
  sas_problem p{};
  p.num_seqs = nseq;
  p.total_tokens = 264;
  p.total_qblocks = 5;
  p.hq = 8;
  p.hkv = 2;
  p.head_dim = 128;
  p.block = 64;
  p.budget_blocks = 4;
  p.dtype = SAS_BF16;
  p.out_dtype = SAS_BF16;
  p.scale = 1.f / std::sqrt(128.f);
  p.cu_seqlens = DI;
  p.cu_qblocks = DI;
  p.cu_seqlens_host = cu;
  p.cu_qblocks_host = cuq;
  p.gate_position = SAS_GATE_INNER;

  expect("gate_topk ok", sas_gate_topk(&p, DF, 4, SAS_GATE_HIST, DI, DF, DF, nullptr), SAS_OK);
  expect("gate_topk ld", sas_gate_topk(&p, DF, 3, SAS_GATE_HIST, DI, DF, DF, nullptr),
         SAS_ERR_SHAPE);
  expect("gate_topk mode", sas_gate_topk(&p, DF, 4, 9, DI, DF, DF, nullptr), SAS_ERR_SHAPE);
  expect("fwd ok", sas_fwd(&p, D, D, D, DI, DF, D, DF, nullptr), SAS_OK);
  expect("fwd null", sas_fwd(&p, nullptr, D, D, DI, DF, D, DF, nullptr), SAS_ERR_NULL);
  expect("fwd align", sas_fwd(&p, (char *)D + 4, D, D, DI, DF, D, DF, nullptr), SAS_ERR_ALIGN);
  const size_t ws = sas_bwd_workspace_size(&p);
  if (ws == 0) { std::printf("FAIL bwd workspace size 0\n"); ++g_failures; }
  expect("bwd ok", sas_bwd(&p, D, D, D, D, D, DF, DI, DF, DF, DF, DF, DF, D, ws, nullptr),
         SAS_OK);
  expect("bwd ws", sas_bwd(&p, D, D, D, D, D, DF, DI, DF, DF, DF, DF, DF, D, ws - 1, nullptr),
         SAS_ERR_WORKSPACE);
  expect("gate_bwd ok", sas_gate_bwd(&p, DF, 4, SAS_GATE_HIST, DI, DF, DF, DF, nullptr), SAS_OK);

  sas_problem q = p;
  q.head_dim = 96;
  expect("head_dim", sas_fwd(&q, D, D, D, DI, DF, D, DF, nullptr), SAS_ERR_UNSUPPORTED);
  q = p;
  q.hq = 6;
  q.hkv = 4;
  expect("groups", sas_fwd(&q, D, D, D, DI, DF, D, DF, nullptr), SAS_ERR_SHAPE);
  q = p;
  q.budget_blocks = 300;
  expect("budget", sas_fwd(&q, D, D, D, DI, DF, D, DF, nullptr), SAS_ERR_UNSUPPORTED);
  q = p;
  q.total_qblocks = 6;
  expect("qblocks", sas_fwd(&q, D, D, D, DI, DF, D, DF, nullptr), SAS_ERR_SHAPE);
  q = p;
  q.scale = NAN;
  expect("scale", sas_fwd(&q, D, D, D, DI, DF, D, DF, nullptr), SAS_ERR_SHAPE);
  q = p;
  q.budget_blocks = 120;
  expect("bwd lds", sas_bwd(&q, D, D, D, D, D, DF, DI, DF, DF, DF, DF, DF, D,
                            sas_bwd_workspace_size(&q), nullptr),
         SAS_ERR_UNSUPPORTED);
  expect("null problem", sas_fwd(nullptr, D, D, D, DI, DF, D, DF, nullptr), SAS_ERR_NULL);

  // -------------------------------------------------- decode problems
  const int batch = 2;
  int32_t *sl = new int32_t[batch]{700, 129};  // 11 and 3 pages
  const int max_pages = 11;
  int32_t *table = new int32_t[batch * max_pages];
  for (int i = 0; i < batch * max_pages; ++i) table[i] = -1;
  for (int c = 0; c < 11; ++c) table[c] = c;
  for (int c = 0; c < 3; ++c) table[max_pages + c] = 11 + c;
  sas_decode_problem d{};
  d.batch = batch;
  d.hq = 8;
  d.hkv = 2;
  d.head_dim = 128;
  d.block = 64;
  d.budget_blocks = 4;
  d.dtype = SAS_BF16;
  d.out_dtype = SAS_BF16;
  d.layout = SAS_KV_PAGED;
  d.max_seqlen = 700;
  d.max_pages = max_pages;
  d.num_pages = 14;
  d.nblk_stride = 64;
  d.scale = 1.f / std::sqrt(128.f);
  d.seqlens = DI;
  d.seqlens_host = sl;
  d.page_table = DI;
  d.summary_dtype = SAS_SUMMARY_F32;
  d.page_table_host = table;
  d.num_splits = 0;
  const size_t dws = sas_decode_workspace_size(&d);
  if (dws == 0) { std::printf("FAIL decode workspace size 0\n"); ++g_failures; }
  expect("pool ok", sas_pool_keys(&d, D, D, nullptr), SAS_OK);
  expect("append ok", sas_decode_append(&d, D, D, D, D, D, nullptr, nullptr), SAS_OK);
  expect("append coarse", sas_decode_append(&d, D, D, D, D, D, D, nullptr), SAS_OK);
  expect("pool coarse", sas_pool_coarse(&d, D, D, nullptr), SAS_OK);
  expect("pool coarse null", sas_pool_coarse(&d, D, nullptr, nullptr), SAS_ERR_NULL);
  const size_t hws = sas_decode_select_hier_workspace_size(&d, 4);
  if (hws == 0) { std::printf("FAIL hier workspace size 0\n"); ++g_failures; }
  expect("hier ok", sas_decode_select_hier(&d, D, D, D, 4, DF, DI, DF, DF, D, hws, nullptr),
         SAS_OK);
  expect("hier ws", sas_decode_select_hier(&d, D, D, D, 4, DF, DI, DF, DF, D, hws - 1, nullptr),
         SAS_ERR_WORKSPACE);
  expect("hier keep 0", sas_decode_select_hier(&d, D, D, D, 0, DF, DI, DF, DF, D, hws, nullptr),
         SAS_ERR_SHAPE);
  expect("hier keep 128",
         sas_decode_select_hier(&d, D, D, D, 128, DF, DI, DF, DF, D, hws, nullptr),
         SAS_ERR_SHAPE);
  expect("hier null", sas_decode_select_hier(&d, D, D, nullptr, 4, DF, DI, DF, DF, D, hws,
                                             nullptr),
         SAS_ERR_NULL);
  const size_t sws = sas_decode_select_workspace_size(&d);
  if (sws == 0) { std::printf("FAIL select workspace size 0\n"); ++g_failures; }
  expect("select ok", sas_decode_select(&d, D, D, DF, DI, DF, DF, D, sws, nullptr), SAS_OK);
  expect("select ws", sas_decode_select(&d, D, D, DF, DI, DF, DF, D, sws - 1, nullptr),
         SAS_ERR_WORKSPACE);
  expect("decode ok", sas_decode(&d, D, D, D, DI, DF, D, DF, D, dws, nullptr), SAS_OK);
  expect("decode noalloc ok", sas_decode_noalloc(&d, D, D, D, DI, DF, D, DF, nullptr), SAS_OK);
  expect("decode ws", sas_decode(&d, D, D, D, DI, DF, D, DF, D, dws - 1, nullptr),
         SAS_ERR_WORKSPACE);
  table[max_pages + 2] = 14;  // past num_pages
  expect("page range", sas_decode(&d, D, D, D, DI, DF, D, DF, D, dws, nullptr), SAS_ERR_SHAPE);
  table[max_pages + 2] = 13;
  table[max_pages + 3] = 99;  // unused entry: not checked
  expect("unused page", sas_decode(&d, D, D, D, DI, DF, D, DF, D, dws, nullptr), SAS_OK);
  sas_decode_problem e = d;
  e.num_splits = 5;
  expect("splits", sas_decode(&e, D, D, D, DI, DF, D, DF, D, dws, nullptr), SAS_ERR_SHAPE);
  e = d;
  e.max_pages = 5;
  expect("max_pages", sas_pool_keys(&e, D, D, nullptr), SAS_ERR_SHAPE);
  e = d;
  e.hq = 6;
  expect("decode group", sas_decode(&e, D, D, D, DI, DF, D, DF, D, dws, nullptr),
         SAS_ERR_UNSUPPORTED);  // groups of 3 heads
  e = d;
  e.nblk_stride = 3;
  expect("stride", sas_decode_select(&e, D, D, DF, DI, DF, DF, D, sws, nullptr), SAS_ERR_SHAPE);
  e.nblk_stride = 70;  // not whole 64-block summary tiles
  expect("stride tiles", sas_decode_select(&e, D, D, DF, DI, DF, DF, D, sws, nullptr),
         SAS_ERR_SHAPE);
  e = d;
  e.summary_dtype = SAS_SUMMARY_FP8;
  expect("fp8 select", sas_decode_select(&e, D, D, DF, DI, DF, DF, D,
                                         sas_decode_select_workspace_size(&e), nullptr),
         SAS_OK);
  e.summary_dtype = 7;
  expect("summary dtype", sas_pool_keys(&e, D, D, nullptr), SAS_ERR_DTYPE);
  e = d;
  e.layout = SAS_KV_CONTIGUOUS;
  e.page_table = nullptr;
  e.page_table_host = nullptr;
  e.max_seqlen = 600;
  expect("capacity", sas_decode(&e, D, D, D, DI, DF, D, DF, D, dws, nullptr), SAS_ERR_SHAPE);
  e = d;
  e.batch = 32;  // 32 rows of seqlens would be read: use a matching array
  int32_t *sl32 = new int32_t[32];
  for (int i = 0; i < 32; ++i) sl32[i] = 6400;
  e.seqlens_host = sl32;
  e.layout = SAS_KV_CONTIGUOUS;
  e.page_table = nullptr;
  e.page_table_host = nullptr;
  e.max_seqlen = 6400;
  e.hq = 32;
  e.hkv = 8;
  e.budget_blocks = 64;
  e.nblk_stride = 128;
  e.num_splits = 64;
  expect("noalloc too big", sas_decode_noalloc(&e, D, D, D, DI, DF, D, DF, nullptr),
         SAS_ERR_WORKSPACE);

  std::printf("%d stand-in launches, %d failures\n", g_launches, g_failures);
  delete[] cu;
  delete[] cuq;
  delete[] sl;
  delete[] sl32;
  delete[] table;
  return g_failures == 0 ? 0 : 1;
}
