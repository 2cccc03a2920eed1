// C ABI of the SAS library: argument checks on the host, then launches.
// Every check runs before any launch, so a rejected call touches nothing.
#include "sas.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "sas_launch.h"

namespace {

thread_local std::string g_last_error;

sas_status fail(sas_status code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

sas_status ok() {
  g_last_error.clear();
  return SAS_OK;
}

sas_status from_hip(hipError_t e, const char *what) {
  if (e == hipSuccess) return ok();
  return fail(SAS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define REQUIRE(cond, code, ...) \
  do {                           \
    if (!(cond)) return fail(code, __VA_ARGS__); \
  } while (0)

// Checks shared by every varlen entry point; fills the largest per-sequence
// block count.
sas_status check_problem(const sas_problem *p, int *max_blocks) {
  REQUIRE(p, SAS_ERR_NULL, "problem is NULL");
  REQUIRE(p->block == 64, SAS_ERR_UNSUPPORTED, "block must be 64 (got %d)", p->block);
  REQUIRE(p->head_dim == 64 || p->head_dim == 128, SAS_ERR_UNSUPPORTED,
          "head_dim must be 64 or 128 (got %d)", p->head_dim);
  REQUIRE(p->hq > 0 && p->hkv > 0, SAS_ERR_SHAPE, "head counts must be positive");
  REQUIRE(p->hq % p->hkv == 0, SAS_ERR_SHAPE, "hq (%d) is not a multiple of hkv (%d)", p->hq,
          p->hkv);
  // tile loads address 64 rows from a uniform base with 32-bit byte offsets
  REQUIRE((long)p->hq * p->head_dim <= (1L << 20), SAS_ERR_UNSUPPORTED,
          "hq * head_dim must be at most 2^20 (got %ld)", (long)p->hq * p->head_dim);
  REQUIRE(p->budget_blocks >= 1 && p->budget_blocks <= sas::kMaxBudget, SAS_ERR_UNSUPPORTED,
          "budget_blocks must be in [1, %d] (got %d)", sas::kMaxBudget, p->budget_blocks);
  REQUIRE(p->dtype == SAS_BF16 || p->dtype == SAS_F32, SAS_ERR_DTYPE, "unknown dtype %d",
          p->dtype);
  REQUIRE(p->out_dtype == SAS_BF16 || p->out_dtype == SAS_F32, SAS_ERR_DTYPE,
          "unknown out_dtype %d", p->out_dtype);
  REQUIRE(!(p->dtype == SAS_F32 && p->out_dtype == SAS_BF16), SAS_ERR_UNSUPPORTED,
          "fp32 inputs need an fp32 output");
  REQUIRE(std::isfinite(p->scale), SAS_ERR_SHAPE, "scale is not finite");
  REQUIRE(p->gate_position == SAS_GATE_INNER || p->gate_position == SAS_GATE_OUTER,
          SAS_ERR_SHAPE, "unknown gate_position %d", p->gate_position);
  REQUIRE(p->num_seqs >= 1, SAS_ERR_SHAPE, "num_seqs must be >= 1");
  REQUIRE(p->cu_seqlens && p->cu_qblocks, SAS_ERR_NULL, "cu_seqlens / cu_qblocks is NULL");
  REQUIRE(p->cu_seqlens_host && p->cu_qblocks_host, SAS_ERR_NULL,
          "host copies of cu_seqlens / cu_qblocks are required");
  REQUIRE(p->cu_seqlens_host[0] == 0 && p->cu_qblocks_host[0] == 0, SAS_ERR_SHAPE,
          "cu_seqlens[0] and cu_qblocks[0] must be 0");
  int mb = 0;
  for (int s = 0; s < p->num_seqs; ++s) {
    const int len = p->cu_seqlens_host[s + 1] - p->cu_seqlens_host[s];
    REQUIRE(len >= 0, SAS_ERR_SHAPE, "cu_seqlens decreases at sequence %d", s);
    const int nb = (len + 63) / 64;
    REQUIRE(p->cu_qblocks_host[s + 1] - p->cu_qblocks_host[s] == nb, SAS_ERR_SHAPE,
            "cu_qblocks[%d..%d] does not match ceil(len / 64) = %d", s, s + 1, nb);
    if (nb > mb) mb = nb;
  }
  REQUIRE(p->cu_seqlens_host[p->num_seqs] == p->total_tokens, SAS_ERR_SHAPE,
          "total_tokens (%d) != cu_seqlens[num_seqs] (%d)", p->total_tokens,
          p->cu_seqlens_host[p->num_seqs]);
  REQUIRE(p->cu_qblocks_host[p->num_seqs] == p->total_qblocks, SAS_ERR_SHAPE,
          "total_qblocks (%d) != cu_qblocks[num_seqs] (%d)", p->total_qblocks,
          p->cu_qblocks_host[p->num_seqs]);
  if (max_blocks) *max_blocks = mb;
  return SAS_OK;
}

}  // namespace

extern "C" {

int32_t sas_abi_version(void) { return SAS_ABI_VERSION; }

const char *sas_status_string(sas_status s) {
  switch (s) {
    case SAS_OK: return "ok";
    case SAS_ERR_NULL: return "a required pointer is NULL";
    case SAS_ERR_SHAPE: return "inconsistent sizes";
    case SAS_ERR_DTYPE: return "unknown dtype";
    case SAS_ERR_ALIGN: return "tensor not 16-byte aligned";
    case SAS_ERR_UNSUPPORTED: return "unsupported configuration";
    case SAS_ERR_WORKSPACE: return "workspace missing or too small";
    case SAS_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char *sas_last_error(void) { return g_last_error.c_str(); }

sas_status sas_gate_topk(const sas_problem *p, const float *logits, int64_t ld,
                         int32_t gate_mode, int32_t *sel_idx, float *sel_loggate,
                         float *gate_lse, void *stream) {
  int mb = 0;
  sas_status st = check_problem(p, &mb);
  if (st) return st;
  REQUIRE(logits && sel_idx && sel_loggate && gate_lse, SAS_ERR_NULL,
          "logits / sel_idx / sel_loggate / gate_lse is NULL");
  REQUIRE(gate_mode >= SAS_GATE_HIST && gate_mode <= SAS_GATE_STE, SAS_ERR_SHAPE,
          "unknown gate_mode %d", gate_mode);
  REQUIRE(ld >= mb && ld >= 1, SAS_ERR_SHAPE, "ld (%lld) < blocks of the longest sequence (%d)",
          (long long)ld, mb);
  sas::GateParams g{};
  g.scores = logits;
  g.ld = ld;
  g.QB = p->total_qblocks;
  g.num_seqs = p->num_seqs;
  g.hkv = p->hkv;
  g.cu_qblocks = p->cu_qblocks;
  g.Kb = p->budget_blocks;
  g.mode = gate_mode;
  g.sel_idx = sel_idx;
  g.sel_lg = sel_loggate;
  g.gate_lse = gate_lse;
  g.nrows = p->hkv * p->total_qblocks;
  return from_hip(sas::launch_gate_topk(g, (hipStream_t)stream), "gate_topk launch");
}

sas_status sas_fwd(const sas_problem *p, const void *q, const void *k, const void *v,
                   const int32_t *sel_idx, const float *sel_loggate, void *o, float *lse,
                   void *stream) {
  sas_status st = check_problem(p, nullptr);
  if (st) return st;
  REQUIRE(q && k && v && sel_idx && sel_loggate && o && lse, SAS_ERR_NULL,
          "a tensor argument of sas_fwd is NULL");
  REQUIRE(aligned16(q) && aligned16(k) && aligned16(v) && aligned16(o), SAS_ERR_ALIGN,
          "q, k, v and o must be 16-byte aligned");
  if (p->total_qblocks == 0) return ok();
  sas::FwdParams f{};
  f.q = q;
  f.k = k;
  f.v = v;
  f.sel_idx = sel_idx;
  f.sel_lg = sel_loggate;
  f.o = o;
  f.lse = lse;
  f.cu_seqlens = p->cu_seqlens;
  f.cu_qblocks = p->cu_qblocks;
  f.num_seqs = p->num_seqs;
  f.T = p->total_tokens;
  f.QB = p->total_qblocks;
  f.hq = p->hq;
  f.hkv = p->hkv;
  f.G = p->hq / p->hkv;
  f.Kb = p->budget_blocks;
  f.scale_log2 = p->scale * 1.4426950408889634f;
  f.outer = p->gate_position == SAS_GATE_OUTER;
  return from_hip(sas::launch_fwd(f, p->dtype == SAS_BF16, p->out_dtype == SAS_BF16,
                                  p->head_dim, (hipStream_t)stream),
                  "fwd launch");
}

sas_status sas_gate_bwd(const sas_problem *p, const float *logits, int64_t ld,
                        int32_t gate_mode, const int32_t *sel_idx, const float *gate_lse,
                        const float *d_loggate, float *d_logits, void *stream) {
  int mb = 0;
  sas_status st = check_problem(p, &mb);
  if (st) return st;
  REQUIRE(logits && sel_idx && gate_lse && d_loggate && d_logits, SAS_ERR_NULL,
          "a tensor argument of sas_gate_bwd is NULL");
  REQUIRE(gate_mode >= SAS_GATE_HIST && gate_mode <= SAS_GATE_STE, SAS_ERR_SHAPE,
          "unknown gate_mode %d", gate_mode);
  REQUIRE(ld >= mb && ld >= 1, SAS_ERR_SHAPE, "ld (%lld) < blocks of the longest sequence (%d)",
          (long long)ld, mb);
  sas::GateBwdParams g{};
  g.logits = logits;
  g.ld = ld;
  g.QB = p->total_qblocks;
  g.num_seqs = p->num_seqs;
  g.hkv = p->hkv;
  g.Kb = p->budget_blocks;
  g.mode = gate_mode;
  g.cu_qblocks = p->cu_qblocks;
  g.sel_idx = sel_idx;
  g.gate_lse = gate_lse;
  g.dlg = d_loggate;
  g.dlogits = d_logits;
  g.nrows = p->hkv * p->total_qblocks;
  return from_hip(sas::launch_gate_bwd(g, (hipStream_t)stream), "gate_bwd launch");
}

namespace {

constexpr int kSeg = 64;  // keeping rows per dk/dv segment (at most 64)

struct BwdLayout {
  size_t off_L, off_D, off_dO16, off_list, off_count, off_segoff, off_dlgpart,
      off_partial, total;
  int U, nhc, max_nb;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

BwdLayout bwd_layout(const sas_problem *p, int max_nb) {
  BwdLayout L{};
  const size_t nx = (size_t)p->hkv * p->total_qblocks;
  const int G = p->hq / p->hkv;
  const int nw = G >= 4 ? 4 : (G >= 2 ? 2 : 1);
  L.nhc = (G + nw - 1) / nw;
  L.max_nb = max_nb > 0 ? max_nb : 1;
  // segments: sum over key blocks of max(1, ceil(count / kSeg)), count <= kept entries
  L.U = (int)((nx * p->budget_blocks + kSeg - 1) / kSeg + nx);
  size_t off = 0;
  const size_t rows = (size_t)p->hq * p->total_qblocks * 64;  // per-block padded rows
  L.off_L = off;        off = align256(off + 16 * rows);  // 16-byte row records
  L.off_D = off;        off = align256(off + 16 * rows);
  L.off_dO16 = off;     // bf16 copy of an fp32 dO for the dk/dv phase
  if (p->dtype == SAS_BF16 && p->out_dtype == SAS_F32)
    off = align256(off + 2 * (size_t)p->total_tokens * p->hq * p->head_dim);
  L.off_list = off;     off = align256(off + sizeof(int32_t) * nx * L.max_nb);
  L.off_count = off;    off = align256(off + sizeof(int32_t) * nx);
  L.off_segoff = off;   off = align256(off + sizeof(int32_t) * (nx + 1));
  L.off_dlgpart = off;
  if (L.nhc > 1) off = align256(off + sizeof(float) * L.nhc * nx * p->budget_blocks);
  L.off_partial = off;  off = align256(off + sizeof(float) * (size_t)L.U * 2 * 64 * p->head_dim);
  L.total = off;
  return L;
}

// Checks shared by the backward phases; fills the kernel parameters.
sas_status bwd_setup(const sas_problem *p, void *workspace, size_t workspace_bytes,
                     sas::BwdParams *b) {
  int mb = 0;
  sas_status st = check_problem(p, &mb);
  if (st) return st;
  REQUIRE(p->total_qblocks < (1 << 23), SAS_ERR_UNSUPPORTED,
          "total_qblocks must be below 2^23 (got %d)", p->total_qblocks);
  const BwdLayout L = bwd_layout(p, mb);
  REQUIRE(workspace, SAS_ERR_WORKSPACE, "workspace is NULL (needs %zu bytes)", L.total);
  REQUIRE(workspace_bytes >= L.total, SAS_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu",
          workspace_bytes, L.total);
  REQUIRE(aligned16(workspace), SAS_ERR_ALIGN, "workspace must be 16-byte aligned");
  char *ws = static_cast<char *>(workspace);
  *b = sas::BwdParams{};
  b->cu_seqlens = p->cu_seqlens;
  b->cu_qblocks = p->cu_qblocks;
  b->num_seqs = p->num_seqs;
  b->T = p->total_tokens;
  b->QB = p->total_qblocks;
  b->hq = p->hq;
  b->hkv = p->hkv;
  b->G = p->hq / p->hkv;
  b->Kb = p->budget_blocks;
  b->max_nb = L.max_nb;
  b->scale = p->scale;
  b->scale_log2 = p->scale * 1.4426950408889634f;
  b->outer = p->gate_position == SAS_GATE_OUTER;
  b->Lbuf = reinterpret_cast<float *>(ws + L.off_L);
  b->Dbuf = reinterpret_cast<float *>(ws + L.off_D);
  b->dO16 = (p->dtype == SAS_BF16 && p->out_dtype == SAS_F32)
                ? reinterpret_cast<__bf16 *>(ws + L.off_dO16) : nullptr;
  b->list = reinterpret_cast<int32_t *>(ws + L.off_list);
  b->count = reinterpret_cast<int32_t *>(ws + L.off_count);
  b->seg_off = reinterpret_cast<int32_t *>(ws + L.off_segoff);
  b->dlg_part = reinterpret_cast<float *>(ws + L.off_dlgpart);
  b->partial = reinterpret_cast<float *>(ws + L.off_partial);
  b->seg = kSeg;
  b->U = L.U;
  return SAS_OK;
}

}  // namespace

size_t sas_bwd_workspace_size(const sas_problem *p) {
  int mb = 0;
  if (check_problem(p, &mb) != SAS_OK) return 0;
  return bwd_layout(p, mb).total;
}

sas_status sas_bwd_prepare(const sas_problem *p, const int32_t *sel_idx, void *workspace,
                           size_t workspace_bytes, void *stream) {
  sas::BwdParams b;
  sas_status st = bwd_setup(p, workspace, workspace_bytes, &b);
  if (st) return st;
  REQUIRE(sel_idx, SAS_ERR_NULL, "sel_idx is NULL");
  if (p->total_qblocks == 0) return ok();
  b.sel_idx = sel_idx;
  return from_hip(sas::launch_bwd_prepare(b, (hipStream_t)stream), "bwd prepare launch");
}

sas_status sas_bwd_dq(const sas_problem *p, const void *q, const void *k, const void *v,
                      const void *o, const void *dO, const float *lse, const int32_t *sel_idx,
                      const float *sel_loggate, float *dq, float *d_loggate, void *workspace,
                      size_t workspace_bytes, void *stream) {
  sas::BwdParams b;
  sas_status st = bwd_setup(p, workspace, workspace_bytes, &b);
  if (st) return st;
  REQUIRE(q && k && v && o && dO && lse && sel_idx && sel_loggate && dq && d_loggate,
          SAS_ERR_NULL, "a tensor argument of sas_bwd_dq is NULL");
  REQUIRE(aligned16(q) && aligned16(k) && aligned16(v) && aligned16(o) && aligned16(dO) &&
              aligned16(dq),
          SAS_ERR_ALIGN, "q, k, v, o, dO and dq must be 16-byte aligned");
  REQUIRE(sas::bwd_dq_supported(b, p->dtype == SAS_BF16, p->head_dim), SAS_ERR_UNSUPPORTED,
          "budget_blocks %d too large for the backward's LDS at this head_dim / dtype",
          p->budget_blocks);
  if (p->total_qblocks == 0) return ok();
  b.q = q;
  b.k = k;
  b.v = v;
  b.o = o;
  b.dO = dO;
  b.lse = lse;
  b.sel_idx = sel_idx;
  b.sel_lg = sel_loggate;
  b.dq = dq;
  b.dlg = d_loggate;
  return from_hip(sas::launch_bwd_dq(b, p->dtype == SAS_BF16, p->out_dtype == SAS_BF16,
                                     p->head_dim, (hipStream_t)stream),
                  "bwd dq launch");
}

sas_status sas_bwd_dkdv(const sas_problem *p, const void *q, const void *k, const void *v,
                        const void *dO, const float *lse, const float *sel_loggate, float *dk,
                        float *dv, void *workspace, size_t workspace_bytes, void *stream) {
  sas::BwdParams b;
  sas_status st = bwd_setup(p, workspace, workspace_bytes, &b);
  if (st) return st;
  REQUIRE(q && k && v && dO && lse && sel_loggate && dk && dv, SAS_ERR_NULL,
          "a tensor argument of sas_bwd_dkdv is NULL");
  REQUIRE(aligned16(q) && aligned16(k) && aligned16(v) && aligned16(dO) && aligned16(dk) &&
              aligned16(dv),
          SAS_ERR_ALIGN, "q, k, v, dO, dk and dv must be 16-byte aligned");
  if (p->total_qblocks == 0) return ok();
  b.q = q;
  b.k = k;
  b.v = v;
  b.dO = dO;
  b.dO_t = b.dO16 ? static_cast<const void *>(b.dO16) : dO;
  b.lse = lse;
  b.sel_lg = sel_loggate;
  b.dk = dk;
  b.dv = dv;
  return from_hip(sas::launch_bwd_dkdv(b, p->dtype == SAS_BF16, p->out_dtype == SAS_BF16,
                                       p->head_dim, (hipStream_t)stream),
                  "bwd dkdv launch");
}

sas_status sas_bwd(const sas_problem *p, const void *q, const void *k, const void *v,
                   const void *o, const void *dO, const float *lse, const int32_t *sel_idx,
                   const float *sel_loggate, float *dq, float *dk, float *dv,
                   float *d_loggate, void *workspace, size_t workspace_bytes, void *stream) {
  sas::BwdParams b;
  sas_status st = bwd_setup(p, workspace, workspace_bytes, &b);
  if (st) return st;
  REQUIRE(q && k && v && o && dO && lse && sel_idx && sel_loggate && dq && dk && dv &&
              d_loggate,
          SAS_ERR_NULL, "a tensor argument of sas_bwd is NULL");
  REQUIRE(aligned16(q) && aligned16(k) && aligned16(v) && aligned16(o) && aligned16(dO) &&
              aligned16(dq) && aligned16(dk) && aligned16(dv),
          SAS_ERR_ALIGN, "q, k, v, o, dO, dq, dk and dv must be 16-byte aligned");
  REQUIRE(sas::bwd_dq_supported(b, p->dtype == SAS_BF16, p->head_dim), SAS_ERR_UNSUPPORTED,
          "budget_blocks %d too large for the backward's LDS at this head_dim / dtype",
          p->budget_blocks);
  st = sas_bwd_prepare(p, sel_idx, workspace, workspace_bytes, stream);
  if (st) return st;
  st = sas_bwd_dq(p, q, k, v, o, dO, lse, sel_idx, sel_loggate, dq, d_loggate, workspace,
                  workspace_bytes, stream);
  if (st) return st;
  return sas_bwd_dkdv(p, q, k, v, dO, lse, sel_loggate, dk, dv, workspace, workspace_bytes,
                      stream);
}

namespace {

sas_status check_decode(const sas_decode_problem *p) {
  REQUIRE(p, SAS_ERR_NULL, "decode problem is NULL");
  REQUIRE(p->block == 64, SAS_ERR_UNSUPPORTED, "block must be 64 (got %d)", p->block);
  REQUIRE(p->head_dim == 64 || p->head_dim == 128, SAS_ERR_UNSUPPORTED,
          "head_dim must be 64 or 128 (got %d)", p->head_dim);
  REQUIRE(p->batch >= 1, SAS_ERR_SHAPE, "batch must be >= 1");
  REQUIRE(p->hq > 0 && p->hkv > 0 && p->hq % p->hkv == 0, SAS_ERR_SHAPE,
          "hq (%d) must be a positive multiple of hkv (%d)", p->hq, p->hkv);
  const int G = p->hq / p->hkv;
  REQUIRE(G == 1 || G == 2 || G == 4 || G == 8, SAS_ERR_UNSUPPORTED,
          "decode supports query groups of 1, 2, 4 or 8 heads (got %d)", G);
  REQUIRE(p->budget_blocks >= 1 && p->budget_blocks <= sas::kMaxBudget, SAS_ERR_UNSUPPORTED,
          "budget_blocks must be in [1, %d] (got %d)", sas::kMaxBudget, p->budget_blocks);
  REQUIRE(p->dtype == SAS_BF16, SAS_ERR_DTYPE, "decode takes bf16 q and caches");
  REQUIRE(p->out_dtype == SAS_BF16 || p->out_dtype == SAS_F32, SAS_ERR_DTYPE,
          "unknown out_dtype %d", p->out_dtype);
  REQUIRE(p->layout == SAS_KV_CONTIGUOUS || p->layout == SAS_KV_PAGED, SAS_ERR_SHAPE,
          "unknown layout %d", p->layout);
  REQUIRE(std::isfinite(p->scale), SAS_ERR_SHAPE, "scale is not finite");
  REQUIRE(p->summary_dtype == SAS_SUMMARY_F32 || p->summary_dtype == SAS_SUMMARY_BF16 ||
              p->summary_dtype == SAS_SUMMARY_FP8,
          SAS_ERR_DTYPE, "unknown summary_dtype %d", p->summary_dtype);
  REQUIRE(p->seqlens && p->seqlens_host, SAS_ERR_NULL, "seqlens (device and host) required");
  int maxL = 0;
  for (int b = 0; b < p->batch; ++b) {
    REQUIRE(p->seqlens_host[b] >= 1, SAS_ERR_SHAPE, "seqlens[%d] = %d < 1", b,
            p->seqlens_host[b]);
    if (p->seqlens_host[b] > maxL) maxL = p->seqlens_host[b];
  }
  if (p->layout == SAS_KV_CONTIGUOUS) {
    REQUIRE(p->max_seqlen >= maxL, SAS_ERR_SHAPE, "max_seqlen (%d) < longest sequence (%d)",
            p->max_seqlen, maxL);
  } else {
    REQUIRE(p->page_table, SAS_ERR_NULL, "paged layout needs a page table");
    REQUIRE(p->max_pages >= (maxL + 63) / 64, SAS_ERR_SHAPE,
            "max_pages (%d) < pages of the longest sequence (%d)", p->max_pages,
            (maxL + 63) / 64);
    REQUIRE(p->num_pages >= 1, SAS_ERR_SHAPE, "num_pages must be >= 1");
    if (p->page_table_host) {
      for (int b = 0; b < p->batch; ++b) {
        const int32_t *row = p->page_table_host + (long)b * p->max_pages;
        const int used = (p->seqlens_host[b] + 63) / 64;
        for (int c = 0; c < used; ++c)
          REQUIRE(row[c] >= 0 && row[c] < p->num_pages, SAS_ERR_SHAPE,
                  "page_table[%d][%d] = %d is outside [0, num_pages = %d)", b, c, row[c],
                  p->num_pages);
      }
    }
  }
  REQUIRE(p->num_splits >= 0 && p->num_splits <= p->budget_blocks, SAS_ERR_SHAPE,
          "num_splits (%d) must be in [0, budget_blocks = %d]", p->num_splits,
          p->budget_blocks);
  REQUIRE(p->nblk_stride >= 1 && p->nblk_stride % 64 == 0, SAS_ERR_SHAPE,
          "nblk_stride (%d) must be a positive multiple of 64 (whole summary tiles)",
          p->nblk_stride);
  REQUIRE(p->nblk_stride >= (maxL - 1) / 64, SAS_ERR_SHAPE,
          "nblk_stride (%d) < history blocks of the longest sequence (%d)", p->nblk_stride,
          (maxL - 1) / 64);
  return SAS_OK;
}

// Compute units of the current device, queried once per device (256 when
// there is no device to ask: the value only shapes the decode split).
int device_cu_count() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cached[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return 256;
  }
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n <= 0) {
    (void)hipGetLastError();
    n = 256;
  }
  cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Split of every row's kept blocks over workgroups.  Automatic: a
// workgroup's 4 waves each stream every 4th block of its split, and as many
// workgroups as the device's compute units hold at once (the attend
// kernel's residency per unit) keep it streaming in a single round, with at
// least one block per wave in a split.
void decode_split(const sas_decode_problem *p, int cu_count, int *nsplit_out,
                  int *per_split_out) {
  const int rows = p->batch * p->hkv;
  int nsplit = p->num_splits;
  if (nsplit == 0) {
    const int max_split = (p->budget_blocks + 3) / 4;
    const int target = cu_count * sas::kDecodeWgPerCu;
    nsplit = (target + rows - 1) / rows;
    if (nsplit > max_split) nsplit = max_split;
    if (nsplit < 1) nsplit = 1;
  }
  const int per_split = (p->budget_blocks + nsplit - 1) / nsplit;
  *per_split_out = per_split;
  *nsplit_out = (p->budget_blocks + per_split - 1) / per_split;
}

// super-block summaries per row: nblk_stride / 8 rounded up to whole tiles
int coarse_stride(const sas_decode_problem *p) {
  return (p->nblk_stride / sas::kCoarseBlocks + 63) / 64 * 64;
}

sas::DecodeParams decode_params(const sas_decode_problem *p) {
  sas::DecodeParams d{};
  d.seqlens = p->seqlens;
  d.page_table = p->page_table;
  d.paged = p->layout == SAS_KV_PAGED;
  d.max_pages = p->max_pages;
  d.max_seqlen = p->max_seqlen;
  d.batch = p->batch;
  d.hq = p->hq;
  d.hkv = p->hkv;
  d.D = p->head_dim;
  d.Kb = p->budget_blocks;
  d.nblk_stride = p->nblk_stride;
  d.sum_kind = p->summary_dtype == SAS_SUMMARY_BF16  ? sas::kSumBf16
               : p->summary_dtype == SAS_SUMMARY_FP8 ? sas::kSumFp8
                                                     : sas::kSumF32;
  d.sqrt_d = sqrtf((float)p->head_dim);
  d.scale_log2 = p->scale * 1.4426950408889634f;
  d.out_bf16 = p->out_dtype == SAS_BF16;
  decode_split(p, p->num_splits ? 0 : device_cu_count(), &d.nsplit, &d.per_split);
  d.coarse_div = 1;
  d.cstride = coarse_stride(p);
  return d;
}

// Partial results of split rows: [rows][nsplit][G][D + 2] fp32.
size_t decode_partial_bytes(const sas_decode_problem *p, int nsplit) {
  return sizeof(float) * (size_t)p->batch * p->hkv * nsplit * (p->hq / p->hkv) *
         (p->head_dim + 2);
}

// Workspace sized from the problem alone: the split asked for, or (automatic
// split) the most splits the library picks on any device.
size_t decode_ws_bytes(const sas_decode_problem *p) {
  int nsplit = 0, per_split = 0;
  decode_split(p, 1 << 30, &nsplit, &per_split);
  return decode_partial_bytes(p, nsplit);
}

// Chunking of the decode selection over workgroups: V blocks per thread
// (256 V blocks per chunk).  One block per thread keeps every thread's
// summary requests in flight at once; V grows (up to 8) only while the
// row's merge would take more than 4096 candidates (chunks x (Kb - 1)).
struct SelectGeom {
  int v, nchunk, nt;  // blocks per thread, chunks per row, threads per chunk
};

int summary_bytes(const sas_decode_problem *p) {
  return p->summary_dtype == SAS_SUMMARY_F32 ? 4 : p->summary_dtype == SAS_SUMMARY_BF16 ? 2 : 1;
}

// div = 1: blocks; div = kCoarseBlocks: super-blocks (kh = kept per row)
SelectGeom select_geom(const sas_decode_problem *p, int div = 1, int kh = 0) {
  int maxhist = 1;
  for (int b = 0; b < p->batch; ++b) {
    const int n = ((p->seqlens_host[b] - 1) / 64) / div;
    if (n > maxhist) maxhist = n;
  }
  if (kh <= 0) kh = p->budget_blocks > 1 ? p->budget_blocks - 1 : 1;
  const long rows = (long)p->batch * p->hkv;
  auto chunks = [&](int nt, int v) { return (maxhist + nt * v - 1) / (nt * v); };
  // 512-thread chunks (half the workgroups and of the merge's candidates)
  // when 256-thread ones would put more than two workgroups on each of 256
  // compute units, for 1- or 2-byte summaries: measured faster for the
  // many-row paged batch, slower for a few long rows
  if (summary_bytes(p) < 4 && rows * chunks(256, 1) > 512 && chunks(512, 1) * kh <= 4096)
    return {1, chunks(512, 1), 512};
  int v = 1;
  while (v < 8 && chunks(256, v) * kh > 4096) v *= 2;
  return {v, chunks(256, v), 256};
}


constexpr int kMaxSelectCandidates = 4096;

// [rows][nchunk][Kb - 1] candidates | [rows][nchunk] (max, sum)
size_t select_ws_bytes(const sas_decode_problem *p, const SelectGeom &sg) {
  const size_t n = (size_t)p->batch * p->hkv * sg.nchunk;
  return align256(n * (p->budget_blocks - 1) * sizeof(int2)) + n * sizeof(float2);
}

}  // namespace

size_t sas_decode_select_workspace_size(const sas_decode_problem *p) {
  if (check_decode(p) != SAS_OK) return 0;
  return select_ws_bytes(p, select_geom(p));
}

size_t sas_decode_workspace_size(const sas_decode_problem *p) {
  if (check_decode(p) != SAS_OK) return 0;
  return decode_ws_bytes(p);
}

sas_status sas_pool_keys(const sas_decode_problem *p, const void *k_cache, void *ksum,
                         void *stream) {
  sas_status st = check_decode(p);
  if (st) return st;
  REQUIRE(k_cache && ksum, SAS_ERR_NULL, "k_cache / ksum is NULL");
  REQUIRE(aligned16(k_cache), SAS_ERR_ALIGN, "k_cache must be 16-byte aligned");
  sas::DecodeParams d = decode_params(p);
  d.k = k_cache;
  d.ksum = ksum;
  return from_hip(sas::launch_pool_keys(d, (hipStream_t)stream), "pool_keys launch");
}

sas_status sas_pool_coarse(const sas_decode_problem *p, const void *ksum, void *csum,
                           void *stream) {
  sas_status st = check_decode(p);
  if (st) return st;
  REQUIRE(ksum && csum, SAS_ERR_NULL, "ksum / csum is NULL");
  REQUIRE(aligned16(ksum) && aligned16(csum), SAS_ERR_ALIGN,
          "ksum and csum must be 16-byte aligned");
  sas::DecodeParams d = decode_params(p);
  d.ksum = const_cast<void *>(ksum);
  d.csum = csum;
  return from_hip(sas::launch_pool_coarse(d, (hipStream_t)stream), "pool_coarse launch");
}

sas_status sas_decode_append(const sas_decode_problem *p, const void *k_new, const void *v_new,
                             void *k_cache, void *v_cache, void *ksum, void *csum,
                             void *stream) {
  sas_status st = check_decode(p);
  if (st) return st;
  REQUIRE(k_new && v_new && k_cache && v_cache && ksum, SAS_ERR_NULL,
          "a tensor argument of sas_decode_append is NULL");
  REQUIRE(!csum || aligned16(csum), SAS_ERR_ALIGN, "csum must be 16-byte aligned");
  sas::DecodeParams d = decode_params(p);
  d.ksum = ksum;
  d.csum = csum;
  return from_hip(sas::launch_decode_append(d, k_new, v_new, k_cache, v_cache,
                                            (hipStream_t)stream),
                  "decode_append launch");
}

sas_status sas_decode_select(const sas_decode_problem *p, const void *q, const void *ksum,
                             float *scores, int32_t *sel_idx, float *sel_loggate,
                             float *gate_lse, void *workspace, size_t workspace_bytes,
                             void *stream) {
  sas_status st = check_decode(p);
  if (st) return st;
  REQUIRE(q && ksum && scores && sel_idx && sel_loggate && gate_lse, SAS_ERR_NULL,
          "a tensor argument of sas_decode_select is NULL");
  REQUIRE(aligned16(ksum), SAS_ERR_ALIGN, "ksum must be 16-byte aligned");
  const SelectGeom sg = select_geom(p);
  REQUIRE(sg.nchunk * (p->budget_blocks - 1) <= kMaxSelectCandidates, SAS_ERR_UNSUPPORTED,
          "history of %d chunks x %d kept blocks exceeds the selection's %d candidates",
          sg.nchunk, p->budget_blocks - 1, kMaxSelectCandidates);
  const size_t need = select_ws_bytes(p, sg);
  REQUIRE(workspace && workspace_bytes >= need, SAS_ERR_WORKSPACE,
          "workspace has %zu bytes, needs %zu", workspace ? workspace_bytes : 0, need);
  REQUIRE(aligned16(workspace), SAS_ERR_ALIGN, "workspace must be 16-byte aligned");
  sas::DecodeParams d = decode_params(p);
  d.q = q;
  d.ksum = const_cast<void *>(ksum);
  d.scores = scores;
  sas::SelectParams s{};
  s.nchunk = sg.nchunk;
  s.chunk_v = sg.v;
  s.chunk_threads = sg.nt;
  s.sel_idx = sel_idx;
  s.sel_lg = sel_loggate;
  s.gate_lse = gate_lse;
  char *ws = static_cast<char *>(workspace);
  const size_t n = (size_t)p->batch * p->hkv * sg.nchunk;
  s.cand = reinterpret_cast<int2 *>(ws);
  s.part = reinterpret_cast<float2 *>(ws + align256(n * (p->budget_blocks - 1) * sizeof(int2)));
  return from_hip(sas::launch_decode_select(d, s, (hipStream_t)stream), "decode select launch");
}

namespace {

constexpr int kMaxCoarseKeep = 127;  // 8 C + 7 candidates <= 1024 in the fine pass

// [rows][nchunk][C] coarse candidates | [rows][nchunk] (max, sum) |
// [rows][C + 1] kept super-blocks | [rows][C + 1] their log gates (unused) |
// [rows] coarse lse (unused) | [rows][cstride] coarse scores
struct HierLayout {
  size_t cand, part, kept, kept_lg, kept_lse, cscores, total;
};

HierLayout hier_layout(const sas_decode_problem *p, const SelectGeom &sg, int C) {
  const size_t rows = (size_t)p->batch * p->hkv, n = rows * sg.nchunk;
  HierLayout l{};
  l.cand = 0;
  l.part = l.cand + align256(n * C * sizeof(int2));
  l.kept = l.part + align256(n * sizeof(float2));
  l.kept_lg = l.kept + align256(rows * (C + 1) * sizeof(int32_t));
  l.kept_lse = l.kept_lg + align256(rows * (C + 1) * sizeof(float));
  l.cscores = l.kept_lse + align256(rows * sizeof(float));
  l.total = l.cscores + rows * coarse_stride(p) * sizeof(float);
  return l;
}

}  // namespace

size_t sas_decode_select_hier_workspace_size(const sas_decode_problem *p, int32_t coarse_keep) {
  if (check_decode(p) != SAS_OK || coarse_keep < 1 || coarse_keep > kMaxCoarseKeep) return 0;
  return hier_layout(p, select_geom(p, sas::kCoarseBlocks, coarse_keep), coarse_keep).total;
}

sas_status sas_decode_select_hier(const sas_decode_problem *p, const void *q, const void *ksum,
                                  const void *csum, int32_t coarse_keep, float *scores,
                                  int32_t *sel_idx, float *sel_loggate, float *gate_lse,
                                  void *workspace, size_t workspace_bytes, void *stream) {
  sas_status st = check_decode(p);
  if (st) return st;
  REQUIRE(q && ksum && csum && scores && sel_idx && sel_loggate && gate_lse, SAS_ERR_NULL,
          "a tensor argument of sas_decode_select_hier is NULL");
  REQUIRE(coarse_keep >= 1 && coarse_keep <= kMaxCoarseKeep, SAS_ERR_SHAPE,
          "coarse_keep (%d) must be in [1, %d]", coarse_keep, kMaxCoarseKeep);
  REQUIRE(aligned16(ksum) && aligned16(csum), SAS_ERR_ALIGN,
          "ksum and csum must be 16-byte aligned");
  const SelectGeom sg = select_geom(p, sas::kCoarseBlocks, coarse_keep);
  REQUIRE(sg.nchunk * coarse_keep <= kMaxSelectCandidates, SAS_ERR_UNSUPPORTED,
          "history of %d super-block chunks x %d kept exceeds the selection's %d candidates",
          sg.nchunk, coarse_keep, kMaxSelectCandidates);
  const HierLayout l = hier_layout(p, sg, coarse_keep);
  REQUIRE(workspace && workspace_bytes >= l.total, SAS_ERR_WORKSPACE,
          "workspace has %zu bytes, needs %zu", workspace ? workspace_bytes : 0, l.total);
  REQUIRE(aligned16(workspace), SAS_ERR_ALIGN, "workspace must be 16-byte aligned");
  char *ws = static_cast<char *>(workspace);
  // coarse pass: the chunked selection over super-blocks, coarse_keep kept per row
  sas::DecodeParams c = decode_params(p);
  c.q = q;
  c.ksum = const_cast<void *>(csum);
  c.nblk_stride = c.cstride;
  c.scores = reinterpret_cast<float *>(ws + l.cscores);
  c.Kb = coarse_keep + 1;
  c.coarse_div = sas::kCoarseBlocks;
  sas::SelectParams s{};
  s.nchunk = sg.nchunk;
  s.chunk_v = sg.v;
  s.chunk_threads = sg.nt;
  s.sel_idx = reinterpret_cast<int32_t *>(ws + l.kept);
  s.sel_lg = reinterpret_cast<float *>(ws + l.kept_lg);
  s.gate_lse = reinterpret_cast<float *>(ws + l.kept_lse);
  s.cand = reinterpret_cast<int2 *>(ws + l.cand);
  s.part = reinterpret_cast<float2 *>(ws + l.part);
  st = from_hip(sas::launch_decode_select(c, s, (hipStream_t)stream), "coarse select launch");
  if (st) return st;
  // fine pass over the candidate blocks
  sas::DecodeParams d = decode_params(p);
  d.q = q;
  d.ksum = const_cast<void *>(ksum);
  d.scores = scores;
  sas::HierParams h{};
  h.C = coarse_keep;
  h.kept = s.sel_idx;
  h.sel_idx = sel_idx;
  h.sel_lg = sel_loggate;
  h.gate_lse = gate_lse;
  return from_hip(sas::launch_decode_select_fine(d, h, (hipStream_t)stream),
                  "fine select launch");
}

sas_status sas_decode(const sas_decode_problem *p, const void *q, const void *k_cache,
                      const void *v_cache, const int32_t *sel_idx, const float *sel_loggate,
                      void *o, float *lse, void *workspace, size_t workspace_bytes,
                      void *stream) {
  sas_status st = check_decode(p);
  if (st) return st;
  REQUIRE(q && k_cache && v_cache && sel_idx && o, SAS_ERR_NULL,
          "q, k_cache, v_cache, sel_idx and o are required");
  REQUIRE(aligned16(q) && aligned16(k_cache) && aligned16(v_cache) && aligned16(o),
          SAS_ERR_ALIGN, "q, caches and o must be 16-byte aligned");
  const size_t need = decode_ws_bytes(p);
  REQUIRE(workspace && workspace_bytes >= need, SAS_ERR_WORKSPACE,
          "workspace has %zu bytes, needs %zu", workspace ? workspace_bytes : 0, need);
  REQUIRE(aligned16(workspace), SAS_ERR_ALIGN, "workspace must be 16-byte aligned");
  sas::DecodeParams d = decode_params(p);
  d.q = q;
  d.k = k_cache;
  d.v = v_cache;
  d.sel_idx = sel_idx;
  d.sel_lg = sel_loggate;
  d.o = o;
  d.lse = lse;
  d.partial = static_cast<float *>(workspace);
  return from_hip(sas::launch_decode_attend(d, (hipStream_t)stream), "decode launch");
}

sas_status sas_decode_noalloc(const sas_decode_problem *p, const void *q, const void *k_cache,
                              const void *v_cache, const int32_t *sel_idx,
                              const float *sel_loggate, void *o, float *lse, void *stream) {
  sas_status st = check_decode(p);
  if (st) return st;
  REQUIRE(q && k_cache && v_cache && sel_idx && o, SAS_ERR_NULL,
          "q, k_cache, v_cache, sel_idx and o are required");
  REQUIRE(aligned16(q) && aligned16(k_cache) && aligned16(v_cache) && aligned16(o),
          SAS_ERR_ALIGN, "q, caches and o must be 16-byte aligned");
  sas::DecodeParams d = decode_params(p);
  d.partial = nullptr;
  if (d.nsplit > 1) {  // one split per row writes o and lse directly
    const size_t need = decode_partial_bytes(p, d.nsplit);
    REQUIRE(need <= sas::kDecodeScratchBytes, SAS_ERR_WORKSPACE,
            "split partials need %zu bytes, the fixed scratch holds %zu (use sas_decode "
            "with a workspace, or fewer splits)", need, sas::kDecodeScratchBytes);
    hipError_t e = sas::decode_scratch_address(&d.partial);
    if (e != hipSuccess) return from_hip(e, "decode scratch address");
  }
  d.q = q;
  d.k = k_cache;
  d.v = v_cache;
  d.sel_idx = sel_idx;
  d.sel_lg = sel_loggate;
  d.o = o;
  d.lse = lse;
  return from_hip(sas::launch_decode_attend(d, (hipStream_t)stream), "decode launch");
}

}  // extern "C"
