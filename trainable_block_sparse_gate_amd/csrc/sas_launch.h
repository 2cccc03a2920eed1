// Internal launch interface between the C ABI (sas_api.cpp) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sas {

constexpr int kMaxBudget = 256;  // largest budget_blocks a row may hold
constexpr int kDecodeWgPerCu = 1;  // decode workgroups resident per compute unit

struct GateParams {
  // Row layout: r = g * QB + Q with the query block Q of sequence s at
  // local index i = Q - cu_qblocks[s].
  const float *scores;
  int64_t ld;
  int QB, num_seqs, hkv;
  const int32_t *cu_qblocks;
  int Kb, mode;
  int32_t *sel_idx;
  float *sel_lg;
  float *gate_lse;
  int nrows;
};
hipError_t launch_gate_topk(const GateParams &p, hipStream_t stream);

struct GateBwdParams {
  const float *logits;
  int64_t ld;
  int QB, num_seqs, hkv, Kb, mode;
  const int32_t *cu_qblocks;
  const int32_t *sel_idx;
  const float *gate_lse;
  const float *dlg;
  float *dlogits;
  int nrows;
};
hipError_t launch_gate_bwd(const GateBwdParams &p, hipStream_t stream);

struct FwdParams {
  const void *q, *k, *v;
  const int32_t *sel_idx;
  const float *sel_lg;
  void *o;
  float *lse;
  const int32_t *cu_seqlens, *cu_qblocks;
  int num_seqs, T, QB, hq, hkv, G, Kb;
  float scale_log2;  // softmax scale * log2(e)
  int outer;         // gate position: 0 inside the softmax, 1 on the values
};
hipError_t launch_fwd(const FwdParams &p, int dtype_bf16, int out_bf16, int head_dim,
                      hipStream_t stream);

struct BwdParams {
  const void *q, *k, *v, *o, *dO;
  const float *lse;
  const int32_t *sel_idx;
  const float *sel_lg;
  float *dq, *dk, *dv, *dlg;
  const int32_t *cu_seqlens, *cu_qblocks;
  int num_seqs, T, QB, hq, hkv, G, Kb, max_nb;
  float scale, scale_log2;
  const void *dO_t;  // dO in the input dtype: dO itself, or dO16 when dO is wider
  // workspace carve-up
  // [hq][QB][64] per query row, 16 bytes each: -lse / scale (-inf past a
  // block's end) and -D (D = sum_u P dP exactly; 0 past the end); fp32 inputs
  // use the first 4 bytes as a float, bf16 inputs a [hi, mid, lo, 0 x 5]
  // bf16 record of the value
  float *Lbuf;
  float *Dbuf;
  __bf16 *dO16;      // [T][hq][D] dO rounded to bf16 (bf16 inputs, fp32 dO), else NULL
  // key blocks are indexed x = kb * hkv + g (key-block major)
  int32_t *list;     // [QB*hkv][max_nb]  (query block << 8 | slot) per key block
  int32_t *count;    // [QB*hkv]
  int32_t *seg_off;  // [QB*hkv + 1] prefix sum of segments per key block
  float *dlg_part;   // [nhc][hkv*QB][Kb] when a row's heads span workgroups
  float *partial;    // [U][2][64][D] partial dK / dV of split key blocks
  int seg;           // keeping rows per segment
  int U;             // upper bound on the number of segments (dk/dv grid)
  int outer;         // gate position: 0 inside the softmax, 1 on the values
};
hipError_t launch_bwd_prepare(const BwdParams &p, hipStream_t stream);
bool bwd_dq_supported(const BwdParams &p, int dtype_bf16, int head_dim);
hipError_t launch_bwd_dq(const BwdParams &p, int dtype_bf16, int out_bf16, int head_dim,
                         hipStream_t stream);
hipError_t launch_bwd_dkdv(const BwdParams &p, int dtype_bf16, int out_bf16, int head_dim,
                           hipStream_t stream);

struct DecodeParams {
  const void *q, *k, *v;       // q [batch][hq][D]; caches in either layout
  const int32_t *seqlens;      // [batch]
  const int32_t *page_table;   // [batch][max_pages] when paged
  int paged, max_pages, max_seqlen;
  int batch, hq, hkv, D, Kb, nblk_stride;
  void *ksum;                  // [batch][hkv][nblk_stride/64][D/EPP][64][EPP] (EPP = 16 / element size), fp32, bf16 or fp8
  int sum_kind;                // kSumF32, kSumBf16 or kSumFp8
  float *scores;               // [batch][hkv][nblk_stride]
  float sqrt_d;                // sqrtf(D), for the pooled score
  const int32_t *sel_idx;      // [batch*hkv][Kb]
  const float *sel_lg;         // [batch*hkv][Kb] or NULL
  void *o;                     // [batch][hq][D]
  float *lse;                  // [batch][hq] or NULL
  float scale_log2;
  int out_bf16;
  int nsplit, per_split;       // split-K geometry
  float *partial;              // [batch*hkv][nsplit][G][D + 2]
  // hierarchical selection: super-block summaries (the tiled layout with
  // cstride super-blocks per row), NULL when not kept; coarse_div = 8 when
  // the selection kernels run over super-blocks, else 1
  void *csum;
  int cstride, coarse_div;
};
constexpr int kCoarseBlocks = 8;  // history blocks per super-block
// decode selection (pooled scores -> gate + Top-K) over chunks of each row:
// scores and an exact local Top-K per chunk, then a merge per row
struct SelectParams {
  int nchunk, chunk_v;         // chunks per row; blocks per thread
  int chunk_threads;           // threads per chunk (256, or 512 with chunk_v 1 and
                               // 1- or 2-byte summaries); chunk = chunk_threads chunk_v
  int32_t *sel_idx;            // out [batch*hkv][Kb]
  float *sel_lg;               // out [batch*hkv][Kb]
  float *gate_lse;             // out [batch*hkv]
  int2 *cand;                  // workspace [rows][nchunk][Kb - 1]: (block, score bits)
  float2 *part;                // workspace [rows][nchunk]: chunk max, sum of exp
};
constexpr int kSumF32 = 0, kSumBf16 = 1, kSumFp8 = 2;
hipError_t launch_decode_select(const DecodeParams &p, const SelectParams &s,
                                hipStream_t stream);
// hierarchical selection: the coarse pass (launch_decode_select over the
// super-block summaries, C kept per row into `kept`) and the fine pass
struct HierParams {
  int C;                       // super-blocks kept per row
  const int32_t *kept;         // [batch*hkv][C + 1]: kept super-blocks ascending
  int32_t *sel_idx;            // out [batch*hkv][Kb]
  float *sel_lg;               // out [batch*hkv][Kb]
  float *gate_lse;             // out [batch*hkv]
};
hipError_t launch_decode_select_fine(const DecodeParams &p, const HierParams &h,
                                     hipStream_t stream);
hipError_t launch_pool_coarse(const DecodeParams &p, hipStream_t stream);
hipError_t launch_pool_keys(const DecodeParams &p, hipStream_t stream);
hipError_t launch_decode_append(const DecodeParams &p, const void *k_new, const void *v_new,
                               void *k_cache, void *v_cache, hipStream_t stream);
hipError_t launch_decode_attend(const DecodeParams &p, hipStream_t stream);
// The fixed device scratch sas_decode_noalloc puts split partials in: its
// address on the current device (looked up once per device).
constexpr size_t kDecodeScratchBytes = size_t(4) << 20;
hipError_t decode_scratch_address(float **out);

}  // namespace sas
