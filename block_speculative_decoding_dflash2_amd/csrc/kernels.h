// Kernel argument blocks and host launchers (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dfl {

constexpr int kMaxGroups = 8;

// Per-row RMSNorm factor applied in a GEMM epilogue: row m is multiplied by
// 1 / sqrt(sum_c sumsq[m][c] * inv_width + eps).  sumsq == null: factor 1.
struct RowScale {
  const float* sumsq; int blocks; float inv_width; float eps;
};

// Consumer applied in the GEMM epilogue instead of writing partial sums
// (LDS-tiled path with one K split: each block owns whole output values).
enum { EPI_NONE = 0, EPI_SWIGLU = 1, EPI_QKV = 2 };
struct GemmEpi {
  int kind;
  // EPI_SWIGLU: act[m][f] = SiLU(gate) * up, gate = output column f, up = F + f
  void* act_out; int F;
  // EPI_QKV: RoPE on q and k heads (position ctx_lens[m / bs] + m % bs);
  // q -> q_out [M][nq][d], k -> k_layer rows, v -> v_layer rows (transposed)
  const int32_t* ctx_lens; int bs, nq, nkv, d, Lmax; float theta;
  void* q_out; void* k_layer; void* v_layer;
};

// y[s][m][n] = rowscale[m] * sum_{k in split s} X[m][k] * W[n][k]  (* scale[n])
struct GemmArgs {
  const void* X; int64_t ldx;     // [M][K] act
  const void* W; int64_t ldw;     // [N][K] weight
  const float* scale;             // [N] or null
  float* P; int64_t ldp;          // [splits][M][ldp] float32
  int64_t split_stride;           // elements between splits
  int M, N, K;                    // M = upper bound on rows
  const int32_t* M_dev;           // actual rows = min(*M_dev, M) if set
  int splits, k_split;            // K range per split (multiple of 32)
  RowScale rs;
  // Grouped launch (groups > 1): group g multiplies weight Wg[g] (scale
  // Sg[g]) and writes its partials at P + g * group_stride; grid z = splits * groups.
  int groups;
  const void* Wg[kMaxGroups];
  const float* Sg[kMaxGroups];
  int64_t group_stride;
  GemmEpi epi;                    // EPI_NONE: write partial sums
  int tile_rows;                  // LDS-tiled path: rows per block tile (0: default for M)
};

// Vocabulary ids per block (and per candidate list) of the weight-streaming
// lm_head.
constexpr int kLmGroupIds = 128;

struct LmHeadArgs {
  const void* X; int64_t ldx;     // [M][K] act
  const void* W; int64_t ldw;     // [V][K]
  const float* scale;             // [V] or null
  int M, N, K;                    // N = vocab
  const int32_t* M_dev;
  int groups;                     // ceil(V / kLmGroupIds)
  int k;                          // candidates per group and row
  uint64_t* cand;                 // [M][k][groups] ranking keys (key t of group g at t * groups + g)
  float* debug_logits;            // [M][V] or null
  RowScale rs;
};

struct TopkMergeArgs {
  const uint64_t* cand;           // [M][count]: count / glen sorted lists of glen keys,
  int count, glen, M, k;          //   key j of list g at g * lstride + j * kstride
  int lstride, kstride;
  const int32_t* M_dev;
  int32_t* ids; float* vals;      // [M][k]
  float multiplier, softcap;
};

// Residual / embedding + optional in-block convolution; writes the new
// residual, gain * residual in act dtype and per-column-block sums of squares
// (the RMSNorm factor is applied by the consuming GEMM).
struct NormArgs {
  int H;
  int rows;                       // upper bound on rows
  const int32_t* rows_dev;        // actual rows if set
  int bs;                         // rows per block (conv boundary; 1 = no neighbours)
  // input: embedding mode (embed != null) or residual mode
  const void* embed; const int32_t* anchors; int mask_id; int vocab; float emb_scale;
  const float* base;              // [rows][H] or null
  const float* parts; int splits; int64_t split_stride; int64_t ldp;  // partial sums
  const void* conv; int conv_k;   // [conv_k][H] param or null
  // dynamic taps (conv == null): split-K partial sums of [rows][dgk] taps,
  // tap j of channel c at column (c / dgroup) * conv_k + j; null = none
  const float* dtaps; int dsplits; int64_t dstride; int dgk; int dgroup;
  const void* gain;               // null: n_out = y (no gain)
  float* h_out;                   // [rows][H] float32 or null
  void* n_out;                    // act [out rows][H]: gain * y; row map below
  float* sumsq;                   // [out rows][col_blocks] sums of y^2
  int t_first;                    // slots t < t_first produce no n_out / sumsq row
  // > 0: 1D grid of rows x remap_cb column blocks dealt to the XCDs in
  // contiguous runs (a row and its neighbour rows share an XCD's L2); 0: grid (rows, column blocks)
  int remap_cb;
};

struct QkvEpiArgs {
  const float* parts; int splits; int64_t split_stride; int64_t ldp;  // [S][M][(nq+2nkv)d]
  const int32_t* ctx_lens;
  int M, bs, nq, nkv, d, Lmax;
  float theta;
  void* q_out;                    // [M][nq][d] act
  void* k_layer; void* v_layer;   // cache base of this layer: [Bcap][nkv][Lmax][d], [Bcap][nkv][d][Lmax]
};

struct KvAppendArgs {
  const float* parts; int splits; int64_t split_stride; int64_t ldp;  // per layer [S][Mn][2 nkv d]
  int64_t layer_stride;           // elements between layers' partial blocks
  const int32_t* offsets;         // [B + 1]
  const int32_t* ctx_lens;        // [B]
  int B, Mn, nkv, d, Lmax, nL;
  int64_t cache_layer_stride;     // elements per layer in the caches
  float theta;
  void* k_cache; void* v_cache;
};

struct SwigluArgs {
  const float* parts; int splits; int64_t split_stride; int64_t ldp;  // [S][M][2F]
  int M, F;
  void* out;                      // [M][F] act
};

struct AttnArgs {
  const void* q;                  // [B*bs][nq][d] act
  const void* k_layer; const void* v_layer;
  const int32_t* ctx_lens;
  int B, bs, nq, nkv, d, Lmax, window;
  int chunk_keys, nchunks, qgroups;   // keys per block (multiple of the sub-chunk)
  float* part_o;                  // [B][nkv][nchunks][QS][d]
  float* part_ml;                 // [B][nkv][nchunks][QS][2]
  float scale_log2;
  void* o;                        // [B*bs][nq*d] act, written directly when nchunks == 1
};

struct AttnCombineArgs {
  const float* part_o; const float* part_ml;
  const int32_t* ctx_lens;
  int B, bs, nq, nkv, d, Lmax, window, chunk_keys, nchunks;
  void* o;                        // [B*bs][nq*d] act
};

struct SelectArgs {
  const int32_t* anchors; const int32_t* ids; const float* vals;
  const float* tl; const float* tr;
  int B, P, k, r, V;
  int32_t* path; int32_t* drafts; float* score; float* debug_pair;
  // transition confidence along the path and the draft-length rule
  // (computed when lens or conf is non-null)
  float p_min; int n_min, n_max;
  int32_t* lens; float* conf;
  // Fused candidate merge (cand != null; k <= 16, at most 64 lists per
  // row): before the selector, the block reduces each of its rows' count /
  // glen sorted candidate lists of
  // glen keys (cand [B*P][count], layout as in TopkMergeArgs) to the k
  // best, applies the logit transform and writes them to ids_out /
  // vals_out (the ids / vals read above, same addresses).
  const uint64_t* cand; int count, glen, lstride, kstride;
  float multiplier, softcap;
  int32_t* ids_out; float* vals_out;
};

struct VerifyArgs {
  const int32_t* drafts; const float* logits;
  int B, bs, V, nchunks, chunk;
  uint64_t* part;                 // [B*bs][nchunks]
  int32_t* accepted; int32_t* bonus; int32_t* argmax;
  const int32_t* lens;            // [B] draft lengths, nullable (= bs-1)
  float* draft_prob;              // [B][bs-1] nullable: 1 where the draft is the argmax
};

struct SampleArgs {
  const float* logits; const int32_t* drafts; const int32_t* lens; const float* uni;
  float temp; int top_k; float top_p; float qscale;   // top_k 0 = off, top_p >= 1 = off
  int B, bs, V;
  uint32_t* theta; uint32_t* mkey; uint64_t* S; uint64_t* Ed;   // [B*bs] row results
  int32_t* kept_n; uint32_t* kept_id; uint64_t* kept_w;           // [B*bs], [B*bs][SV_OUT] x2
  int32_t* accepted; int32_t* bonus; float* draft_prob;
};
struct LossArgs {
  const float* logits; const int32_t* labels; const int32_t* anchors;
  const int32_t* ids; const float* vals; const float* tl; const float* tr;
  int B, P, V, k, r, nchunks, chunk;
  float mult, cap, gamma, sel_weight;
  float* part;                    // [B*P][nchunks][2] (max, sum of exp)
  double* seq;                    // [B][6] per-sequence sums
  float* block_ce; float* selector_ce; float* losses;
};
void launch_loss_rows(const LossArgs& a, hipStream_t s);
void launch_loss_seq(const LossArgs& a, hipStream_t s);   // per-sequence sums, then the totals

// Kept sets of at most this many entries are handed from the row pass to the draw.
constexpr int SV_OUT = 256;

// Activation rows above which the LDS-tiled, compute-bound lm_head is used.
constexpr int kTiledMinRows = 64;
// Activation rows above which the linears take the LDS-tiled GEMM: from 33
// rows the weight-streaming kernel holds four activation fragments per k-step
// and keeps one load group in flight (its registers are full), and the tiled
// one streams the weights faster (measured on 60 context rows of the
// long-block workload: context K/V projection 34.8 -> 23.7 us).
constexpr int kTiledMinRowsGemm = 32;

int gemm_rows_per_block(int weight_dtype, int M);
bool gemm_tiled_ok(int weight_dtype, int M, int K);
bool lmhead_tiled_ok(int weight_dtype, int M, int K, int k);
int lmhead_tiled_lists(int weight_dtype, int M, int V);
// Block tile of the LDS-tiled GEMM: bm activation rows x 256 weight rows,
// per_cu blocks resident per CU.  bm = the requested 256, 192 (fp8 weights
// only) or 128 (0: the default for M rows); DFLASH2_TILED_BM overrides it.
struct TiledShape { int bm, per_cu; };
TiledShape tiled_shape(int weight_dtype, int M, int bm);
void launch_gemm_tiled(int weight_dtype, const GemmArgs& a, hipStream_t s);
void launch_lmhead_tiled(int weight_dtype, const LmHeadArgs& a, hipStream_t s);
void launch_gemm(int weight_dtype, const GemmArgs& a, hipStream_t s);
// Whether launch_gemm applies a.epi itself (else the caller runs the
// consumer kernel on the partial sums, which are then written).
bool gemm_epi_fusable(int weight_dtype, const GemmArgs& a);
void launch_lmhead_topk(int weight_dtype, const LmHeadArgs& a, hipStream_t s);
void launch_topk_merge(const TopkMergeArgs& a, hipStream_t s);
// Lists per row after the first fold of `lists` lists (k <= 16), and that
// fold: the 16 best keys of each run of 64 lists, sorted, at
// out[(m * topk_premerge_lists(lists) + c) * 16].
int topk_premerge_lists(int lists);
void launch_topk_premerge(const TopkMergeArgs& a, uint64_t* out, hipStream_t s);
int norm_col_blocks(int H);
void launch_norm(bool f32, const NormArgs& a, hipStream_t s);
void launch_qkv_epilogue(bool f32, const QkvEpiArgs& a, hipStream_t s);
void launch_kv_append(bool f32, const KvAppendArgs& a, hipStream_t s);
void launch_swiglu(bool f32, const SwigluArgs& a, hipStream_t s);
bool attn_supported(int d);
int attn_sub_chunk(bool f32, int d);
void launch_attention(bool f32, const AttnArgs& a, hipStream_t s);
void launch_attn_combine(bool f32, const AttnCombineArgs& a, hipStream_t s);
__host__ __device__ int select_row_stride(int r);
int select_window(int k, int r, int P, size_t budget);
void launch_select(const SelectArgs& a, int tw, hipStream_t s);
void launch_verify_partial(const VerifyArgs& a, hipStream_t s);
void launch_sample_rows(const SampleArgs& a, hipStream_t s);
void launch_sample_pick(const SampleArgs& a, hipStream_t s);
void launch_verify_final(const VerifyArgs& a, hipStream_t s);

}  // namespace dfl
