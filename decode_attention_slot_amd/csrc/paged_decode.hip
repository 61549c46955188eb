// GQA paged decode attention for gfx950.
//
// What is computed ("Padding and Batching with Block KV", sections "Block
// Table", "Cache Masking" and "Multi-Token Decode"; "Decode Context-Length
// Bucketing", sections "Problem" and "Block-table head-trim vs. SWA
// tail-trim"): query token j of request r sits at position L - q_len + j,
// where L counts this step's tokens, and attends to every earlier-or-equal
// position p below walk_blocks * block_size whose block-table entry is
// active; q head h reads KV head h / (Hq / Hkv). The result is the softmax of
// scale * <q, k> over those keys applied to the values, in fp32.
//
// How, on CDNA4:
// * Work unit: one wavefront per (request, chunk of context blocks, KV head).
//   A workgroup holds the waves of up to NW KV heads of one (request,
//   chunk), so the whole [block][token][head][dim] rows a workgroup reads
//   are contiguous in HBM.
// * Chunks are sized on the device from seq_lens (no host synchronisation):
//   about target_pairs (request, chunk) pairs over the batch, at least
//   min_chunk_blocks blocks each, whole blocks, aligned to logical block 0.
//   The split depends only on the context lengths, so a head-trimmed walk,
//   a full-table walk and the context walk produce the same partials.
// * The block ids of a chunk are staged in LDS by the workgroup (pieces of
//   up to 256 blocks), so each tile's block id is an LDS read that does not
//   hold up the vector-memory pipeline.
// * The tile loop is straight-line: the loads of tile t+1 are issued before
//   tile t is computed and are never under a data-dependent branch (an
//   inactive table entry reads null block 0 and is masked; the loop tail
//   re-loads its last tile, which hits in cache), so one tile stays in
//   flight behind the one being computed.
// * Tile of 16 tokens. S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (fp32 KV:
//   v_mfma_f32_16x16x4f32): K is the A operand (lane l holds token l % 16,
//   16 bytes of its head row per piece), Q^T the B operand (lane l holds
//   query row l % 16; rows are (query token, head in group), at most 16).
//   The result gives each lane four tokens of one query row.
// * Online softmax per query row, in exp2 units, entirely inside the lane
//   except one max over the four lane groups.
// * O^T = V^T P^T on v_mfma_f32_16x16x4f32: lane l holds the fp32 value of
//   dimension column l % 16 for token 4 * (l / 16) + i, which is exactly a
//   16-byte slice of that token's head row, so V is read in its natural
//   layout (each 16-lane group reads one whole 256-byte head row). The
//   accumulator lands with query row = l % 16, matching the softmax state.
// * Split-K partials (acc, m, l per row) go to the workspace; the last wave
//   of a (request, KV head) to arrive, found with a device-scope counter,
//   merges them in ascending chunk order and resets the counter.
// * Masked keys are removed by select, never by multiplying by zero, and the
//   values of keys past the context are replaced by -0.0, so unwritten (NaN
//   canary) cache rows cannot leak into the output and a masked product is
//   -0.0, which leaves every accumulator bit-unchanged.
// * The fixed-shape table walk is a separate instantiation: it reads every
//   walked column and folds the bytes it does not need into a sink that is
//   stored only under a flag the host never sets.
#include <math.h>

#include "kvslot_internal.h"

namespace kvs {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr uint32_t kFlagWalkTable = 0x1u;
// Never set by the host. Testing it keeps the table-walk loads alive.
constexpr uint32_t kFlagSink = 0x80000000u;
constexpr int kTile = 16;
constexpr int kStage = 256;  // block ids staged in LDS at a time
constexpr int kSlices = 8;   // 64-request slices of seq_lens kept in registers

__device__ __forceinline__ int wave_sum(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

__device__ __forceinline__ int wave_inclusive_scan(int x, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}

__device__ __forceinline__ float max_over_groups(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

__device__ __forceinline__ float sum_over_groups(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Context positions of a request that a walk of walk_tok positions can see.
__device__ __forceinline__ int visible_len(int L, int walk_tok) {
  return L <= 0 ? 0 : (L < walk_tok ? L : walk_tok);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <bool BF16, int D, int NW, bool TW>
__global__ void __launch_bounds__(NW * 64, 2)
paged_decode_kernel(const DecodeParams p, int bs_shift) {
  constexpr int ES = BF16 ? 2 : 4;       // bytes per element
  constexpr int EP = 16 / ES;            // elements per 16-byte piece
  constexpr int NP = D / (4 * EP);       // 16-byte K pieces per lane per token
  constexpr int NT = D / 16;             // P.V n-tiles (dimension columns of 16)
  constexpr int NVW = NT * ES / 4;       // V dwords per lane per token
  constexpr int PSTRIDE = D + 4;         // floats per partial row (acc, m, l, pad)
  constexpr uint32_t kNegZero = BF16 ? 0x80008000u : 0x80000000u;
  static_assert(NP >= 1 && NVW >= 2, "unsupported head_dim");
  struct TileBuf {
    u32x4 k[NP];         // K pieces of token rho of the tile
    uint32_t v[4][NVW];  // V slices of tokens 4*jg .. 4*jg+3
    int bid;             // block id the tile was read from (<= 0: inactive)
  };
  __shared__ int s_blk[kStage];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int rho = lane & 15;  // query row owned by this lane (MFMA column)
  const int jg = lane >> 4;   // lane group: tokens 4*jg .. 4*jg+3 of a tile

  const int B = p.num_seqs;
  const int bs = 1 << bs_shift;
  const int walk_tok = p.walk_blocks << bs_shift;
  const int Hkv = p.num_kv_heads;
  const int Hq = p.num_q_heads;
  const int G = Hq / Hkv;
  const int Sq = p.q_len;
  const int nrows = G * Sq;
  const int HG = Hkv / NW;  // the launcher picks NW dividing Hkv
  const int64_t block_bytes = ((int64_t)Hkv * D * ES) << bs_shift;
  const uint32_t row_bytes = (uint32_t)(Hkv * D * ES);

  // ---- context blocks of every request ------------------------------------
  // Batches of up to 64 * kSlices requests keep their block counts in
  // registers (lane l of slice k: request 64 k + l), loaded in one round
  // trip, so a workgroup's set-up costs one memory latency.
  const bool in_regs = B <= 64 * kSlices;
  int nbr[kSlices];
#pragma unroll
  for (int k = 0; k < kSlices; ++k) {
    const int rr = 64 * k + lane;
    nbr[k] = 0;
    if (in_regs && rr < B) nbr[k] = (visible_len(p.seq_lens[rr], walk_tok) + bs - 1) >> bs_shift;
  }
  auto blocks_of = [&](int rr) {  // large batches only
    return rr < B ? (visible_len(p.seq_lens[rr], walk_tok) + bs - 1) >> bs_shift : 0;
  };

  // ---- chunk size, from the context blocks of the whole batch ------------
  int64_t ctx_blocks_total = 0;
  if (in_regs) {
    int t = 0;
#pragma unroll
    for (int k = 0; k < kSlices; ++k) t += nbr[k];
    ctx_blocks_total = wave_sum(t);
  } else {
    for (int base = 0; base < B; base += 64) ctx_blocks_total += wave_sum(blocks_of(base + lane));
  }
  int64_t cb64 = (ctx_blocks_total + p.target_pairs - 1) / p.target_pairs;
  if (cb64 < p.min_chunk_blocks) cb64 = p.min_chunk_blocks;
  const int cb = uniform((int)cb64);  // blocks per chunk
  const int chunk_tok = cb << bs_shift;
  const int walk_chunks = (p.walk_blocks + cb - 1) / cb;

  uint32_t sink = 0;

  for (int64_t uw = blockIdx.x;; uw += gridDim.x) {
    const int64_t pair = uw / HG;
    const int hg = (int)(uw - pair * HG);

    // ---- locate (request, chunk) of this pair ----------------------------
    int r = -1, c = 0;
    int64_t pidx0 = 0;  // index of (r, chunk 0) among the pairs that hold context
    if constexpr (!TW) {
      // pair = (sum of chunk counts of requests before r) + c
      int64_t carry = 0;
      auto visit = [&](int base, int nb) {
        const int C = (nb + cb - 1) / cb;
        const int incl = wave_inclusive_scan(C, lane);
        const int tot = __shfl(incl, 63);
        if (r < 0 && pair < carry + tot) {
          const uint64_t hit = __ballot(carry + incl > pair);
          const int src = __builtin_ctzll(hit);
          const int excl = __shfl(incl - C, src);
          r = base + src;
          pidx0 = carry + excl;
          c = (int)(pair - pidx0);
        }
        carry += tot;
      };
      if (in_regs) {
#pragma unroll
        for (int k = 0; k < kSlices; ++k)
          if (64 * k < B) visit(64 * k, nbr[k]);
      } else {
        for (int base = 0; base < B && r < 0; base += 64) visit(base, blocks_of(base + lane));
      }
    } else if (walk_chunks > 0) {
      const int64_t rq = pair / walk_chunks;
      if (rq < B) {
        r = (int)rq;
        c = (int)(pair - rq * walk_chunks);
        int carry = 0;  // chunks holding context of the requests before r
        if (in_regs) {
#pragma unroll
          for (int k = 0; k < kSlices; ++k)
            carry += (64 * k + lane < r) ? (nbr[k] + cb - 1) / cb : 0;
        } else {
          for (int base = 0; base < r; base += 64)
            carry += (base + lane < r) ? (blocks_of(base + lane) + cb - 1) / cb : 0;
        }
        pidx0 = wave_sum(carry);
      }
    }
    // The scan leaves these in vector registers; they are the same in every
    // lane, and saying so keeps the tile loop below under scalar control.
    r = uniform(r);
    c = uniform(c);
    pidx0 = uniform((int)pidx0);  // < target_pairs + num_seqs
    if (r < 0) break;  // every pair is done (uniform over the workgroup)

    const int g = hg * NW + wave;
    const int L = uniform(p.seq_lens[r]);
    const int E = visible_len(L, walk_tok);
    const int nb_r = (E + bs - 1) >> bs_shift;
    const int Cv = (nb_r + cb - 1) / cb;  // chunks of r that hold context
    const bool pair_valid = c < Cv;
    const int tok0 = c * chunk_tok;
    const int tok_valid_end = min(tok0 + chunk_tok, E);
    const int tok_walk_end = TW ? min(tok0 + chunk_tok, walk_tok) : tok_valid_end;

    // ---- query operand (B operand of the score MFMA) ---------------------
    const int jrow = rho / G;
    const int hh = rho - jrow * G;
    const int qpos = rho < nrows ? L - Sq + jrow : -1;
    const int qpos_min = L - Sq;
    u32x4 qp[NP];
    {
      const char* qrow = (const char*)p.q +
                         ((((int64_t)r * Sq + jrow) * Hq + (int64_t)g * G + hh) * D) * ES;
#pragma unroll
      for (int pp = 0; pp < NP; ++pp) {
        qp[pp] = (u32x4){0u, 0u, 0u, 0u};
        if (pair_valid && rho < nrows)
          qp[pp] = *(const u32x4*)(qrow + pp * 64 + jg * 16);
      }
    }

    // ---- running softmax state of query row rho --------------------------
    float m_run = -INFINITY;
    float l_run = 0.0f;  // partial: this lane's tokens only
    f32x4 acc[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[n] = (f32x4){0.f, 0.f, 0.f, 0.f};

    const int32_t* trow = p.block_table + (int64_t)r * p.table_stride;
    const uint32_t k_lane_off = ((uint32_t)rho * Hkv + g) * (D * ES) + jg * 16;
    const uint32_t v_lane_off = ((uint32_t)(4 * jg) * Hkv + g) * (D * ES) + rho * (NT * ES);

    const int blk_first = tok0 >> bs_shift;
    const int blk_end = tok_walk_end > tok0 ? ((tok_walk_end - 1) >> bs_shift) + 1 : blk_first;
    for (int pb = blk_first; pb < blk_end; pb += kStage) {
      const int pn = min(kStage, blk_end - pb);
      __syncthreads();  // the previous piece is consumed by every wave
      for (int i = threadIdx.x; i < pn; i += NW * 64) {
        const int col = pb + i;
        s_blk[i] = col < p.table_stride ? trow[col] : 0;
      }
      __syncthreads();
      const int t_begin = max(tok0, pb << bs_shift);
      const int t_end = min(tok_walk_end, (pb + pn) << bs_shift);
      const int nt = (t_end - t_begin + kTile - 1) / kTile;

      // Loads of one tile: K as the score MFMA's A operand, V in row layout.
      // Always issued: an inactive entry reads null block 0 and is masked.
      auto load = [&](int tt, TileBuf& b) {
        const int bid = uniform(s_blk[(tt >> bs_shift) - pb]);
        const bool active = bid > 0 && (int64_t)bid < p.total_blocks;
        const int64_t base = (int64_t)(active ? bid : 0) * block_bytes;
        const char* kb = (const char*)p.k_cache + base;
        const char* vb = (const char*)p.v_cache + base;
        const uint32_t in_blk = (uint32_t)(tt & (bs - 1)) * row_bytes;
        b.bid = active ? bid : 0;
#pragma unroll
        for (int pp = 0; pp < NP; ++pp)
          b.k[pp] = *(const u32x4*)(kb + in_blk + k_lane_off + pp * 64);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const char* src = vb + in_blk + v_lane_off + i * row_bytes;
          if constexpr (NVW == 2) {
            const u32x2 x = *(const u32x2*)src;
            b.v[i][0] = x[0]; b.v[i][1] = x[1];
          } else {
#pragma unroll
            for (int w = 0; w < NVW; w += 4) {
              const u32x4 x = *(const u32x4*)(src + w * 4);
              b.v[i][w] = x[0]; b.v[i][w + 1] = x[1]; b.v[i][w + 2] = x[2]; b.v[i][w + 3] = x[3];
            }
          }
        }
      };

      // Scores, online softmax and P.V for one tile whose loads have landed.
      auto consume = [&](int tt, TileBuf& b) {
        const bool active = b.bid > 0;
        if constexpr (TW) {
          if (!(pair_valid && active && tt < tok_valid_end)) {
            // Fixed-shape walk past the context: read, never used.
#pragma unroll
            for (int pp = 0; pp < NP; ++pp)
              sink ^= b.k[pp][0] ^ b.k[pp][1] ^ b.k[pp][2] ^ b.k[pp][3];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
              for (int w = 0; w < NVW; ++w) sink ^= b.v[i][w];
            return;
          }
        }

        // ---- scores: S^T[token 4*jg+i][row rho] ----------------------------
        f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int pp = 0; pp < NP; ++pp) {
          if constexpr (BF16) {
            s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, b.k[pp]),
                                                        __builtin_bit_cast(bf16x8, qp[pp]), s,
                                                        0, 0, 0);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              s = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(b.k[pp][e]),
                                                       __uint_as_float(qp[pp][e]), s, 0, 0, 0);
          }
        }

        float sx[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) sx[i] = s[i] * p.scale_log2;
        const bool full = active && (tt + kTile <= tok_valid_end) && (tt + kTile - 1 <= qpos_min);
        if (!full) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int pos = tt + 4 * jg + i;
            const bool kv_ok = active && pos < E;
            if (!(kv_ok && pos <= qpos)) sx[i] = -INFINITY;
            if (!kv_ok) {
#pragma unroll
              for (int w = 0; w < NVW; ++w) b.v[i][w] = kNegZero;
            }
          }
        }

        // ---- online softmax ------------------------------------------------
        float mx = fmaxf(fmaxf(sx[0], sx[1]), fmaxf(sx[2], sx[3]));
        mx = max_over_groups(mx);
        const float m_new = fmaxf(m_run, mx);
        const float m_use = m_new == -INFINITY ? 0.0f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        float pr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) pr[i] = __builtin_amdgcn_exp2f(sx[i] - m_use);
        l_run = l_run * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
        if (__any(alpha != 1.0f)) {
#pragma unroll
          for (int n = 0; n < NT; ++n) acc[n] *= alpha;
        }
        m_run = m_new;

        // ---- O^T += V^T P^T --------------------------------------------------
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
          for (int n = 0; n < NT; ++n) {
            float v;
            if constexpr (BF16) {
              v = (n & 1) ? bf16_hi(b.v[i][n >> 1]) : bf16_lo(b.v[i][n >> 1]);
            } else {
              v = __uint_as_float(b.v[i][n]);
            }
            acc[n] = __builtin_amdgcn_mfma_f32_16x16x4f32(v, pr[i], acc[n], 0, 0, 0);
          }
        }
      };

      // Two tile buffers: tile t+1 is in flight while tile t is computed.
      TileBuf b0, b1;
      load(t_begin, b0);
      for (int t = 0; t < nt; t += 2) {
        const int tt = t_begin + t * kTile;
        load(t + 1 < nt ? tt + kTile : tt, b1);
        consume(tt, b0);
        load(t + 2 < nt ? tt + 2 * kTile : tt, b0);
        if (t + 1 < nt) consume(tt + kTile, b1);
      }
    }

    if (!pair_valid) continue;

    // acc[n][i] holds dimension (4*jg + i) * NT + n of query row rho.
    const float l_tot = sum_over_groups(l_run);
    const int d_base = 4 * jg * NT;

    if (c == 0 && g == 0 && lane == 0) {
      p.chunk_meta[2 * r] = (int32_t)pidx0;  // where request r's partials start
      p.chunk_meta[2 * r + 1] = Cv;          // read by the merge kernel
    }

    if (Cv == 1) {
      if (rho < nrows) {
        const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
        float* o = p.out + (((int64_t)r * Sq + jrow) * Hq + (int64_t)g * G + hh) * D + d_base;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
          for (int n0 = 0; n0 < NT; n0 += 4) {
            f32x4 v = {acc[n0][i] * inv, acc[n0 + 1][i] * inv, acc[n0 + 2][i] * inv,
                       acc[n0 + 3][i] * inv};
            *(f32x4*)(o + i * NT + n0) = v;
          }
        }
      }
      continue;
    }

    // ---- split-K: publish this chunk's partial ----------------------------
    const int64_t pidx = pidx0 + c;
    {
      float* prow = p.partials + ((pidx * Hkv + g) * nrows + rho) * PSTRIDE;
      if (rho < nrows) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
          for (int n0 = 0; n0 < NT; n0 += 4) {
            f32x4 v = {acc[n0][i], acc[n0 + 1][i], acc[n0 + 2][i], acc[n0 + 3][i]};
            *(f32x4*)(prow + d_base + i * NT + n0) = v;
          }
        }
        if (jg == 0) {
          prow[D] = m_run;
          prow[D + 1] = l_tot;
        }
      }
    }
  }

  // ---- requests with no visible context produce zeros --------------------
  {
    const int row_floats = Sq * Hq * D;
    for (int r = blockIdx.x; r < B; r += gridDim.x) {
      if (visible_len(p.seq_lens[r], walk_tok) == 0) {
        float* o = p.out + (int64_t)r * row_floats;
        for (int i = threadIdx.x; i < row_floats; i += NW * 64) o[i] = 0.0f;
        if (threadIdx.x == 0) p.chunk_meta[2 * r + 1] = 0;
      }
    }
  }

  if constexpr (TW) {
    if (p.flags & kFlagSink) p.out[0] = __uint_as_float(sink);
  }
}

// Split-K merge: one workgroup per (request, KV head) whose context was
// split over more than one chunk. Wave w merges chunks w, w + NWC, ... in
// ascending order; the NWC partial states are then merged in wave order
// through LDS. The assignment is fixed, so the result is the same on every
// run and for every walk mode. Lane l of a wave owns output float4s
// l + 64 k (k < KC) of the (row, dimension) block. Fewer float4s per lane
// leave room for more waves, so long contexts (many chunks) merge with
// 16 waves.
template <int KC>
struct MergeShape {
  static constexpr int NWC = KC <= 2 ? 16 : 32 / KC;  // waves per workgroup
  static constexpr int CB = KC == 1 ? 8 : (KC == 2 ? 3 : (KC == 4 ? 2 : 1));  // chunks in flight per wave
};

template <int D, int KC>
__global__ void __launch_bounds__(MergeShape<KC>::NWC * 64)
paged_decode_combine_kernel(const DecodeParams p) {
  constexpr int F4ROW = D / 4;
  constexpr int PSTRIDE = D + 4;
  constexpr int CB = MergeShape<KC>::CB;
  constexpr int NWC = MergeShape<KC>::NWC;
  __shared__ float s_m[NWC][KC * 64];
  __shared__ float s_l[NWC][KC * 64];
  __shared__ f32x4 s_o[NWC][KC * 64];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int B = p.num_seqs;
  const int Hkv = p.num_kv_heads;
  const int Hq = p.num_q_heads;
  const int G = Hq / Hkv;
  const int Sq = p.q_len;
  const int nrows = G * Sq;
  const int f4_total = nrows * F4ROW;

  int roff[KC], moff[KC];
  bool ok[KC];
#pragma unroll
  for (int k = 0; k < KC; ++k) {
    const int f = lane + 64 * k;
    const int row = f / F4ROW;
    ok[k] = f < f4_total;
    roff[k] = row * PSTRIDE + (f - row * F4ROW) * 4;
    moff[k] = row * PSTRIDE + D;
  }

  for (int64_t u = blockIdx.x; u < (int64_t)B * Hkv; u += gridDim.x) {
    const int r = (int)(u / Hkv);
    const int g = (int)(u - (int64_t)r * Hkv);
    const int Cv = p.chunk_meta[2 * r + 1];  // pass 1 records it for every request
    if (Cv <= 1) continue;                    // pass 1 wrote this output directly
    const int64_t pidx0 = p.chunk_meta[2 * r];
    const int64_t cstride = (int64_t)Hkv * nrows * PSTRIDE;
    const float* pbase = p.partials + (pidx0 * Hkv + g) * nrows * PSTRIDE;

    float Mx[KC], Ls[KC];
    f32x4 o[KC];
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      Mx[k] = -INFINITY;
      Ls[k] = 0.0f;
      o[k] = (f32x4){0.f, 0.f, 0.f, 0.f};
    }
    for (int c0 = wave; c0 < Cv; c0 += NWC * CB) {
      f32x4 a[CB][KC];
      f32x2 ml[CB][KC];
#pragma unroll
      for (int j = 0; j < CB; ++j) {
        const int cc = c0 + j * NWC;
        const float* pc = pbase + (int64_t)cc * cstride;
#pragma unroll
        for (int k = 0; k < KC; ++k) {
          if (cc < Cv && ok[k]) {
            a[j][k] = *(const f32x4*)(pc + roff[k]);
            ml[j][k] = *(const f32x2*)(pc + moff[k]);
          }
        }
      }
#pragma unroll
      for (int j = 0; j < CB; ++j) {
#pragma unroll
        for (int k = 0; k < KC; ++k) {
          if (c0 + j * NWC < Cv && ok[k] && ml[j][k][0] != -INFINITY) {
            const float mn = fmaxf(Mx[k], ml[j][k][0]);
            const float so = __builtin_amdgcn_exp2f(Mx[k] - mn);
            const float sn = __builtin_amdgcn_exp2f(ml[j][k][0] - mn);
            Ls[k] = Ls[k] * so + ml[j][k][1] * sn;
            o[k] = o[k] * so + a[j][k] * sn;
            Mx[k] = mn;
          }
        }
      }
    }
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      s_m[wave][lane + 64 * k] = Mx[k];
      s_l[wave][lane + 64 * k] = Ls[k];
      s_o[wave][lane + 64 * k] = o[k];
    }
    __syncthreads();
    for (int f = threadIdx.x; f < f4_total; f += NWC * 64) {
      float M = -INFINITY, Lt = 0.0f;
      f32x4 ot = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < NWC; ++w) {
        const float mw = s_m[w][f];
        if (mw == -INFINITY) continue;
        const float mn = fmaxf(M, mw);
        const float so = __builtin_amdgcn_exp2f(M - mn);
        const float sn = __builtin_amdgcn_exp2f(mw - mn);
        Lt = Lt * so + s_l[w][f] * sn;
        ot = ot * so + s_o[w][f] * sn;
        M = mn;
      }
      const int row = f / F4ROW;
      const int jr = row / G;
      const int hr = row - jr * G;
      const float inv = Lt > 0.0f ? 1.0f / Lt : 0.0f;
      float* orow = p.out + (((int64_t)r * Sq + jr) * Hq + (int64_t)g * G + hr) * D;
      *(f32x4*)(orow + (f - row * F4ROW) * 4) = ot * inv;
    }
    __syncthreads();
  }
}

template <bool BF16, int D, int NW>
hipError_t launch_typed(const DecodeParams& p, int bs_shift, hipStream_t stream) {
  const int HG = p.num_kv_heads / NW;
  // Upper bound on the (request, chunk) pairs, from host-known sizes only:
  // no request has more than ceil(walk_blocks / min_chunk_blocks) chunks,
  // and the context walk never has more than target_pairs + num_seqs.
  const int64_t cpr = (p.walk_blocks + p.min_chunk_blocks - 1) / p.min_chunk_blocks;
  int64_t pairs = (int64_t)p.num_seqs * (cpr > 0 ? cpr : 1);
  if (!(p.flags & kFlagWalkTable) && pairs > (int64_t)p.target_pairs + p.num_seqs)
    pairs = (int64_t)p.target_pairs + p.num_seqs;
  int64_t grid = pairs * HG;
  if (grid < 1) grid = 1;
  if (grid > (1 << 20)) grid = 1 << 20;
  if (p.flags & kFlagWalkTable)
    paged_decode_kernel<BF16, D, NW, true>
        <<<dim3((unsigned)grid), dim3(NW * 64), 0, stream>>>(p, bs_shift);
  else
    paged_decode_kernel<BF16, D, NW, false>
        <<<dim3((unsigned)grid), dim3(NW * 64), 0, stream>>>(p, bs_shift);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int64_t cgrid = (int64_t)p.num_seqs * p.num_kv_heads;
  if (cgrid > 65536) cgrid = 65536;
  const int nrows = p.num_q_heads / p.num_kv_heads * p.q_len;
  const int kc = (nrows * (D / 4) + 63) / 64;
  const dim3 cg((unsigned)cgrid);
#define KVS_MERGE(KC)                                                             \
  paged_decode_combine_kernel<D, KC>                                              \
      <<<cg, dim3(MergeShape<KC>::NWC * 64), 0, stream>>>(p)
  if (kc <= 1) KVS_MERGE(1);
  else if (kc <= 2) KVS_MERGE(2);
  else if (kc <= 4) KVS_MERGE(4);
  else KVS_MERGE(8);
#undef KVS_MERGE
  return hipGetLastError();
}

template <bool BF16, int D>
hipError_t launch_heads(const DecodeParams& p, int bs_shift, hipStream_t stream) {
  const int h = p.num_kv_heads;
  if (h % 8 == 0) return launch_typed<BF16, D, 8>(p, bs_shift, stream);
  if (h % 4 == 0) return launch_typed<BF16, D, 4>(p, bs_shift, stream);
  if (h % 2 == 0) return launch_typed<BF16, D, 2>(p, bs_shift, stream);
  return launch_typed<BF16, D, 1>(p, bs_shift, stream);
}

}  // namespace

int32_t decode_target_pairs(int32_t num_kv_heads) {
  // About 8192 waves of work over the 1024 SIMDs of a 256-CU part, so the
  // (request, chunk) units spread evenly over the CUs.
  const int32_t t = 8192 / (num_kv_heads > 0 ? num_kv_heads : 1);
  return t > 16 ? t : 16;
}

int32_t decode_min_chunk_blocks(int32_t block_size) {
  // At least 128 tokens per chunk keeps the partial traffic a few percent
  // of the KV bytes the chunk reads.
  const int32_t b = 128 / block_size;
  return b > 1 ? b : 1;
}

size_t decode_meta_bytes(int32_t num_seqs) {
  return ((size_t)num_seqs * 2 * sizeof(int32_t) + 255) / 256 * 256;
}

size_t decode_partial_bytes(int32_t num_seqs, int32_t q_len, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t head_dim) {
  const size_t pairs = (size_t)decode_target_pairs(num_kv_heads) + (size_t)num_seqs;
  return pairs * (size_t)num_q_heads * (size_t)q_len * (size_t)(head_dim + 4) * sizeof(float);
}

hipError_t launch_paged_decode(const DecodeParams& p, hipStream_t stream) {
  const int bs_shift = __builtin_ctz((unsigned)p.block_size);
  if (p.is_bf16) {
    if (p.head_dim == 128) return launch_heads<true, 128>(p, bs_shift, stream);
    return launch_heads<true, 64>(p, bs_shift, stream);
  }
  if (p.head_dim == 128) return launch_heads<false, 128>(p, bs_shift, stream);
  return launch_heads<false, 64>(p, bs_shift, stream);
}

}  // namespace kvs
