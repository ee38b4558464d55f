// Multi-query paged attention for gfx950 (MI355X): several causal query tokens
// per sequence over the paged BF16 cache (chunked prefill, multi-token decode).
//
// The query tokens of all sequences are packed token-major, sequence b owning
// rows query_start[b] .. query_start[b+1]-1 ("Qwen3-14B" pypto-lib page,
// prefill_fwd section); they are the last Lq of the sequence's ctx cached
// tokens, so query i sees tokens [0, ctx - Lq + i] (standard causal attention,
// "Qwen 3" TensorSharp docs, section 4.1). A row that sees no token gives
// zeros.
//
// Work decomposition
//   A row is one (query token, query head) pair of one KV head h: row r of
//   sequence b and head h is token r / G, head h*G + r % G. mq_kernel<D,RT,KS>
//   takes one workgroup per (sequence, KV head, block of 16*RT rows, split);
//   its RT*KS waves are RT row tiles of 16 rows times KS KV streams. Each
//   iteration stages KS consecutive 32-token chunks of K and V (one per
//   stream) in LDS, and every wave then works on its stream's chunk:
//   1. S^T = K . Q^T on v_mfma_f32_16x16x32_bf16 (16 tokens x 16 rows per
//      MFMA), so that lane (lq, lr) ends up with 8 scores of row lr: tokens
//      4*lq + i and 16 + 4*lq + i of the chunk, i = 0..3.
//   2. Online softmax per row (max over the 4 lane groups by lane shuffles,
//      lane-local running sums, exp2 of log2-scaled scores).
//   3. O^T += V^T . P^T on the same MFMA: the lane's 8 probabilities, rounded
//      to BF16, are already its B operand (k index 8*lq + j <-> the token of
//      its j-th score); the A operand, V^T, comes from LDS through gfx950's
//      transposing read ds_read_b64_tr_b16, whose lane i of a 16-lane group
//      receives element i % 4 of the 8 bytes addressed by lanes 4j + i / 4,
//      j = 0..3 -- so lanes 4j + c point at 4 dims of the j-th token.
//   The KS streams of a row tile are merged in LDS in a fixed order. With one
//   split the workgroup writes the normalised BF16 output; otherwise it writes
//   the unnormalised FP32 sum, the running max (log2 units) and the sum, and
//   mq_reduce_kernel<D> merges the splits of every row.
//
// The reduction order is fixed (no atomics): repeated calls are bit-identical.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "device_common.h"
#include "launch.h"

namespace pa {
namespace {

constexpr int kMqPage = 128;   // tokens per page
constexpr int kChunk = 32;     // tokens of one stream per iteration

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef char __attribute__((address_space(3))) lds_char;

// KV streams per workgroup for a row-tile count: 4 waves in all, except that
// head_dim 256 with one row tile keeps to 2 streams (64 KiB of LDS).
__host__ __device__ constexpr int mq_streams(int d, int rt) {
  return rt >= 4 ? 1 : (rt == 2 ? 2 : (d == 128 ? 4 : 2));
}

// LDS bytes: K tiles of the KS streams, then their V tiles, each tile 32
// token rows of 2*D bytes. The end-of-kernel stream merge reuses the space.
__host__ __device__ constexpr int mq_lds_bytes(int d, int rt) {
  return 2 * mq_streams(d, rt) * kChunk * 2 * d;
}

// 16-byte chunk c of token row r of a tile is stored at chunk position
// c ^ (r & 15) (K: the 16 lanes of a score-operand read hit 16 different
// positions) or c ^ ((r & 7) << 1) (V: the 8 (row, chunk) pairs of a
// transposing read hit 8 different positions).
template <int D>
__device__ __forceinline__ uint32_t k_off(int r, int c) {
  return (uint32_t)r * (2 * D) + 16u * (uint32_t)(c ^ (r & 15));
}
template <int D>
__device__ __forceinline__ uint32_t v_off(int r, int c) {
  return (uint32_t)r * (2 * D) + 16u * (uint32_t)(c ^ ((r & 7) << 1));
}

__device__ __forceinline__ u32x2 lds_read_tr16(const lds_char* base, uint32_t off) {
  const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (v4i16 __attribute__((address_space(3)))*)(base + off));
  return __builtin_bit_cast(u32x2, r);
}

template <int D, int RT, int KS>
__global__ __launch_bounds__(64 * RT * KS) void mq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_cache,
    const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ context_lens, const int32_t* __restrict__ query_start,
    uint16_t* __restrict__ out, float* __restrict__ ws_acc, float* __restrict__ ws_ml,
    int batch, int num_tokens, int num_kv_heads, int gqa, int max_pages, int num_pages,
    int max_query_len, int row_blocks, int split_pages, int num_splits, float score_scale) {
  static_assert(D == 128 || D == 256, "head_dim");
  constexpr int NT = 64 * RT * KS;          // threads
  constexpr int ROWS = 16 * RT;             // rows per workgroup
  constexpr int KD = D / 32;                // k-steps of the score MFMA
  constexpr int DB = D / 16;                // 16-dim blocks of the output
  constexpr int CPR = D / 8;                // 16-byte chunks per token row
  constexpr int TILE = kChunk * 2 * D;      // bytes of one 32-token tile
  constexpr int UPT = 2 * KS * kChunk * CPR / NT;  // staged chunks per thread
  constexpr int IT = KS * kChunk;           // tokens per iteration
  static_assert(UPT * NT == 2 * KS * kChunk * CPR, "staging must tile evenly");
  static_assert(UPT % 2 == 0, "half K, half V");
  static_assert(mq_lds_bytes(D, RT) == 2 * KS * TILE, "LDS size");

  extern __shared__ __attribute__((aligned(16))) char smem_mq[];
  lds_char* lds = (lds_char*)smem_mq;

  // 1-D grid, (sequence, KV head) pair fastest, then row block, then split.
  const int num_pairs = batch * num_kv_heads;
  const int pair = blockIdx.x % num_pairs;
  const int rest = blockIdx.x / num_pairs;
  const int rb = rest % row_blocks;
  const int s = rest / row_blocks;
  const int h = pair % num_kv_heads;
  const int b = pair / num_kv_heads;
  const int num_q_heads = num_kv_heads * gqa;

  // A sequence whose query range is not inside [0, num_tokens] or is longer
  // than max_query_len is skipped: its rows are not written.
  const int qs0 = query_start[b];
  const int lqn = query_start[b + 1] - qs0;
  if (qs0 < 0 || lqn <= 0 || lqn > max_query_len || qs0 > num_tokens - lqn) return;
  const int rows_b = lqn * gqa;
  const int row0 = rb * ROWS;
  if (row0 >= rows_b) return;
  const int ctx = context_lens[b];
  const bool bad_ctx = ctx < 0 || ctx > max_pages * kMqPage;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rt = wave % RT;   // row tile
  const int g = wave / RT;    // KV stream
  const int lq = lane >> 4;
  const int lr = lane & 15;

  // This lane's row (lr of the tile) and the tokens it may see.
  const int row = row0 + 16 * rt + lr;
  const bool row_ok = row < rows_b;
  const int i_tok = row_ok ? row / gqa : 0;
  const int hq = h * gqa + (row_ok ? row - i_tok * gqa : 0);
  const size_t t_row = (size_t)qs0 + i_tok;  // packed token index of the row

  const int split_tokens = split_pages * kMqPage;
  const int t_begin = s * split_tokens;
  const int last_row = min(row0 + ROWS, rows_b) - 1;
  const int n_last = bad_ctx ? 0 : ctx - lqn + last_row / gqa + 1;
  const int t_end = min(t_begin + split_tokens, n_last);
  if (num_splits > 1 && (bad_ctx || t_end <= t_begin)) return;  // the merge skips it
  const int n_row = ctx - lqn + i_tok + 1;
  const int lim = row_ok ? min(n_row, t_end) : 0;  // tokens [t_begin, lim) are visible

  // B operand of the score MFMA: lane (lq, lr) holds dims 32*kk + 8*lq .. +7
  // of its row's q, the dims its K operand holds (zeros for rows past the end).
  u32x4 qb[KD];
  {
    const uint16_t* qrow = q + (t_row * num_q_heads + hq) * D;
#pragma unroll
    for (int kk = 0; kk < KD; ++kk)
      qb[kk] = row_ok ? load16(qrow + 32 * kk + 8 * lq) : u32x4{0u, 0u, 0u, 0u};
  }

  // ---- staging: chunk k of thread tid is unit u = tid + NT*k; units
  // [0, NT*UPT/2) are K, the rest V; in each half, unit -> (stream, row, chunk).
  const size_t page_elems = (size_t)kMqPage * num_kv_heads * D;
  const size_t row_elems = (size_t)num_kv_heads * D;
  const int32_t* bt_row = block_table + (size_t)b * max_pages;
  const int n_it = t_end > t_begin ? (t_end - t_begin + IT - 1) / IT : 0;

  u32x4 stg[UPT];
  int stg_tb = 0;        // first token of the staged iteration
  bool stg_bad = false;  // its page id is outside the pool
  int next_page = n_it > 0 ? bt_row[t_begin / kMqPage] : 0;

  auto issue = [&](int it) {
    const int tb = t_begin + it * IT;
    const int page = next_page;
    if (it + 1 < n_it) next_page = bt_row[(tb + IT) / kMqPage];
    stg_tb = tb;
    stg_bad = (unsigned)page >= (unsigned)num_pages;
    const size_t base = (size_t)(stg_bad ? 0 : page) * page_elems + (size_t)h * D +
                        (size_t)(tb & (kMqPage - 1)) * row_elems;
#pragma unroll
    for (int k = 0; k < UPT; ++k) {
      const int u = (tid + NT * k) % (NT * UPT / 2);
      const int c = u % CPR;
      const int tr = u / CPR;  // token of the iteration: stream * 32 + row
      const uint16_t* pool = k < UPT / 2 ? k_cache : v_cache;
      stg[k] = load16(pool + base + (size_t)tr * row_elems + 8 * c);
    }
  };
  auto commit = [&]() {
#pragma unroll
    for (int k = 0; k < UPT; ++k) {
      const bool is_k = k < UPT / 2;
      const int u = (tid + NT * k) % (NT * UPT / 2);
      const int c = u % CPR;
      const int tr = u / CPR;
      const int st = tr / kChunk;
      const int r = tr % kChunk;
      u32x4 v = stg[k];
      // rows past the range hold other data (NaN poison included): zero them,
      // so that P = 0 times V stays 0. A bad page reads as NaN K (the rows
      // that see it become NaN) and zero V (the rows that do not see it are
      // unaffected).
      if (stg_tb + tr >= t_end) v = u32x4{0u, 0u, 0u, 0u};
      else if (stg_bad) v = is_k ? u32x4{0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u}
                                 : u32x4{0u, 0u, 0u, 0u};
      const uint32_t off = (is_k ? 0u : (uint32_t)(KS * TILE)) + (uint32_t)(st * TILE) +
                           (is_k ? k_off<D>(r, c) : v_off<D>(r, c));
      *(u32x4 __attribute__((address_space(3)))*)(lds + off) = v;
    }
  };

  // ---- running state of the lane's row ------------------------------------
  float m_run = -INFINITY;  // max of the log2-scaled scores seen
  float l_run = 0.f;        // lane-local part of the sum of probabilities
  f32x4 o[DB];              // O^T: lane (lq, lr) holds dims 16*db + 4*lq + i of row lr
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  const lds_char* kt = lds + g * TILE;
  const lds_char* vt = lds + KS * TILE + g * TILE;

  auto compute = [&](int it) {
    const int tb = t_begin + it * IT + kChunk * g;  // first token of this stream's chunk
    f32x4 sacc[2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      sacc[half] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KD; ++kk) {
        const u32x4 a =
            *(const u32x4 __attribute__((address_space(3)))*)(kt + k_off<D>(16 * half + lr, 4 * kk + lq));
        sacc[half] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, qb[kk]), sacc[half], 0, 0, 0);
      }
    }
    // lane (lq, lr): sacc[half][i] = S[row lr][token tb + 16*half + 4*lq + i]
    float sc[8];
    float mx = -INFINITY;
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = tb + 16 * half + 4 * lq + i;
        const float v = t < lim ? sacc[half][i] * score_scale : -INFINITY;
        sc[4 * half + i] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    f32x8 p;
#pragma unroll
    for (int j = 0; j < 8; ++j) p[j] = fast_exp2(sc[j] - m_use);
    const bf16x8 pb = __builtin_convertvector(p, bf16x8);
    float ps = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) ps += (float)pb[j];  // the sum of the weights used
    l_run = fmaf(l_run, alpha, ps);
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      o[db] *= alpha;
      // A operand: lane (lq, lr) gets V[token 4*lq + j][16*db + lr] (j < 4)
      // and V[token 16 + 4*lq + j - 4][16*db + lr] (j >= 4).
      const int c = 2 * db + ((lr & 3) >> 1);
      const uint32_t sub = 8u * (lr & 1);
      const u32x2 lo = lds_read_tr16(vt, v_off<D>(4 * lq + (lr >> 2), c) + sub);
      const u32x2 hi = lds_read_tr16(vt, v_off<D>(16 + 4 * lq + (lr >> 2), c) + sub);
      const u32x4 a = u32x4{lo[0], lo[1], hi[0], hi[1]};
      o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), pb, o[db],
                                                      0, 0, 0);
    }
  };

  if (n_it > 0) issue(0);
  for (int it = 0; it < n_it; ++it) {
    __syncthreads();  // every wave is done with the previous tiles
    commit();
    if (it + 1 < n_it) issue(it + 1);
    __syncthreads();
    compute(it);
  }

  // the row's sum over the 4 lane groups (same order on every lane)
  {
    const float l1 = l_run + __shfl_xor(l_run, 16);
    l_run = l1 + __shfl_xor(l1, 32);
  }

  // ---- merge the KS streams of each row tile, in stream order ------------
  if constexpr (KS > 1) {
    constexpr int REC = 32 + 16 * D;  // floats per (row tile, stream): m, l, O^T
    float* rec = (float*)smem_mq;
    __syncthreads();  // every wave is done with the tiles
    if (g > 0) {
      float* my = rec + (size_t)((g - 1) * RT + rt) * REC;
      if (lq == 0) {
        my[lr] = m_run;
        my[16 + lr] = l_run;
      }
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) my[32 + (16 * db + 4 * lq + i) * 16 + lr] = o[db][i];
    }
    __syncthreads();
    if (g > 0) return;
#pragma unroll
    for (int gg = 1; gg < KS; ++gg) {
      const float* ot = rec + (size_t)((gg - 1) * RT + rt) * REC;
      const float m2 = ot[lr];
      const float l2 = ot[16 + lr];
      const float m_new = fmaxf(m_run, m2);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float a1 = fast_exp2(m_run - m_use);
      const float a2 = fast_exp2(m2 - m_use);
      l_run = l_run * a1 + l2 * a2;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          o[db][i] = o[db][i] * a1 + ot[32 + (16 * db + 4 * lq + i) * 16 + lr] * a2;
      m_run = m_new;
    }
  }

  if (!row_ok) return;
  const size_t orow = t_row * num_q_heads + hq;
  if (num_splits == 1) {
    if (bad_ctx) {
      const float nan = __builtin_nanf("");
#pragma unroll
      for (int db = 0; db < DB; ++db)
        store_bf16x4(out + orow * D + 16 * db + 4 * lq, f32x4{nan, nan, nan, nan});
      return;
    }
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;  // no visible token: zeros
#pragma unroll
    for (int db = 0; db < DB; ++db)
      store_bf16x4(out + orow * D + 16 * db + 4 * lq, o[db] * inv);
  } else {
    const size_t slot = orow * num_splits + s;
#pragma unroll
    for (int db = 0; db < DB; ++db)
      *reinterpret_cast<f32x4*>(ws_acc + slot * D + 16 * db + 4 * lq) = o[db];
    if (lq == 0) *reinterpret_cast<float2*>(ws_ml + slot * 2) = make_float2(m_run, l_run);
  }
}

// Merge of the splits of every (query token, query head) row: one thread per 4
// dims. The row's sequence is found by binary search in query_start.
template <int D>
__global__ __launch_bounds__(256) void mq_reduce_kernel(
    const float* __restrict__ ws_acc, const float* __restrict__ ws_ml,
    const int32_t* __restrict__ context_lens, const int32_t* __restrict__ query_start,
    uint16_t* __restrict__ out, int batch, int num_tokens, int num_q_heads, int max_query_len,
    int num_splits, int split_tokens, int max_ctx) {
  constexpr int TPR = D / 4;
  constexpr int RPW = 256 / TPR;
  const int row = blockIdx.x * RPW + (int)threadIdx.x / TPR;
  if (row >= num_tokens * num_q_heads) return;
  const int d4 = ((int)threadIdx.x % TPR) * 4;
  const int t = row / num_q_heads;
  // last b with query_start[b] <= t
  int lo = 0, hi = batch;  // answer in [0, batch)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (query_start[mid] <= t) lo = mid;
    else hi = mid;
  }
  const int qs0 = query_start[lo];
  const int lqn = query_start[lo + 1] - qs0;
  if (qs0 < 0 || lqn <= 0 || lqn > max_query_len || qs0 > num_tokens - lqn) return;
  if (t < qs0 || t >= qs0 + lqn) return;  // not covered by a sequence
  const int ctx = context_lens[lo];
  f32x4 res;
  if (ctx < 0 || ctx > max_ctx) {
    const float nan = __builtin_nanf("");
    res = f32x4{nan, nan, nan, nan};
  } else {
    const int n_row = ctx - lqn + (t - qs0) + 1;
    int nv = n_row <= 0 ? 0 : (n_row + split_tokens - 1) / split_tokens;
    nv = nv > num_splits ? num_splits : nv;
    res = merge_row<D>(ws_acc, ws_ml, (size_t)row, num_splits, nv, d4);
  }
  store_bf16x4(out + (size_t)row * D + d4, res);
}

template <int D, int RT>
int launch_mq_drt(const MqLaunchArgs& a) {
  constexpr int KS = mq_streams(D, RT);
  hipStream_t stream = reinterpret_cast<hipStream_t>(a.stream);
  const int gqa = a.num_q_heads / a.num_kv_heads;
  const dim3 grid(a.batch * a.num_kv_heads * a.row_blocks * a.num_splits);
  void* args[] = {(void*)&a.q,           (void*)&a.k_cache,       (void*)&a.v_cache,
                  (void*)&a.block_table, (void*)&a.context_lens,  (void*)&a.query_start,
                  (void*)&a.out,         (void*)&a.ws_acc,        (void*)&a.ws_ml,
                  (void*)&a.batch,       (void*)&a.num_tokens,    (void*)&a.num_kv_heads,
                  (void*)&gqa,           (void*)&a.max_pages,     (void*)&a.num_pages,
                  (void*)&a.max_query_len, (void*)&a.row_blocks,  (void*)&a.split_pages,
                  (void*)&a.num_splits,  (void*)&a.score_scale};
  return (int)hipLaunchKernel(reinterpret_cast<const void*>(&mq_kernel<D, RT, KS>), grid,
                              dim3(64 * RT * KS), args, mq_lds_bytes(D, RT), stream);
}

template <int D>
int launch_mq_d(const MqLaunchArgs& a) {
  switch (a.row_tiles) {
    case 1: return launch_mq_drt<D, 1>(a);
    case 2: return launch_mq_drt<D, 2>(a);
    default: return launch_mq_drt<D, 4>(a);
  }
}

template <int D>
int launch_mq_reduce_d(const MqLaunchArgs& a) {
  hipStream_t stream = reinterpret_cast<hipStream_t>(a.stream);
  const int rows = a.num_tokens * a.num_q_heads;
  const int split_tokens = a.split_pages * kMqPage;
  const int max_ctx = a.max_pages * kMqPage;
  constexpr int RPW = 256 / (D / 4);
  void* args[] = {(void*)&a.ws_acc,        (void*)&a.ws_ml,       (void*)&a.context_lens,
                  (void*)&a.query_start,   (void*)&a.out,         (void*)&a.batch,
                  (void*)&a.num_tokens,    (void*)&a.num_q_heads, (void*)&a.max_query_len,
                  (void*)&a.num_splits,    (void*)&split_tokens,  (void*)&max_ctx};
  return (int)hipLaunchKernel(reinterpret_cast<const void*>(&mq_reduce_kernel<D>),
                              dim3((rows + RPW - 1) / RPW), dim3(256), args, 0, stream);
}

}  // namespace

int mq_row_tiles(int rows_per_head) { return rows_per_head <= 16 ? 1 : (rows_per_head <= 32 ? 2 : 4); }

int launch_mq(const MqLaunchArgs& a) {
  return a.head_dim == 128 ? launch_mq_d<128>(a) : launch_mq_d<256>(a);
}

int launch_mq_reduce(const MqLaunchArgs& a) {
  return a.head_dim == 128 ? launch_mq_reduce_d<128>(a) : launch_mq_reduce_d<256>(a);
}

}  // namespace pa
