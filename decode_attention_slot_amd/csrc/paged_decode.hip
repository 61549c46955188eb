// GQA paged decode attention for gfx950: the split-K merge, the host-side
// sizes and the launch of one call (pass 1, then the merge). Pass 1 and the
// design of both kernels are described in paged_decode.h.
#include "paged_decode.h"

namespace kvs {
namespace {

// Split-K merge. A request whose context was cut into C > 1 segments has C
// partial states per (KV head, row): (m, l, acc), m the running max in log2
// units, l and acc the sums of exp2(score - m) and of its products with the
// values. The merged output is defined by one fixed association, so it does
// not depend on the launch shape, the batch around the request (padding with
// dummy requests included) or the walk mode:
// * NG logical groups (NG fixed by the row count and head_dim); group j
//   merges partials j, j + NG, j + 2 NG, ... in that order, starting empty;
// * the output merges group states 0 .. NG - 1 in that order, starting empty.
// When C <= NG every group holds at most one partial, a state merged into an
// empty state comes back unchanged, and the definition reduces to merging
// partials 0 .. C - 1 in order. The kernel uses that for units with few
// partials (C <= CS, all loads in flight at once): one wave merges them, each
// lane its own float4, sequentially, with no LDS and no barrier. Other units
// take the grouped path (one wave per group, group states through LDS).
// Either path gives the defined result; the threshold only picks the faster.
// Every output float4 is merged on its own, so a unit (request, KV head) is
// cut into column pieces of 64 KCW float4s (KCW per lane) that separate
// workgroups merge: with KCW = 1 a long context's partials are read by as
// many compute units as the unit has 64-float4 columns. A workgroup owns a
// tile of T consecutive pieces; neither KCW nor T changes a result.

// Merge the state (m, l, o) into the running state (M, Lt, ot). The one merge
// step of every path, with the rounding pinned by explicit fma.
__device__ __forceinline__ void merge_state(float& M, float& Lt, f32x4& ot, float m, float l,
                                            f32x4 o) {
  if (m == -INFINITY) return;  // a state that saw no key
  const float mn = fmaxf(M, m);
  const float so = __builtin_amdgcn_exp2f(M - mn);
  const float sn = __builtin_amdgcn_exp2f(m - mn);
  Lt = __builtin_fmaf(Lt, so, l * sn);
#pragma unroll
  for (int e = 0; e < 4; ++e) ot[e] = __builtin_fmaf(ot[e], so, o[e] * sn);
  M = mn;
}

// Logical groups NG of a unit made of `pieces` columns of 64 float4s (1 to 8):
// 8 up to four pieces, 4 beyond. (16 groups for one- and two-column units
// merged 1 us slower on the 12-request and bucketing workloads: the launch
// of 1024-thread workgroups costs more than the extra partials in flight
// gain; 4 groups for four-column units doubled the 256-request merge, and
// 16 made that call 730 instead of 680 us and its 2-KV-head share 217
// instead of 206 us.)
__host__ __device__ constexpr int merge_groups(int pieces) {
  return pieces <= 4 ? 8 : 4;
}

// KCW: float4s per lane of a piece (a piece is KCW columns of 64 float4s).
template <int D, int NG, int KCW>
__global__ void __launch_bounds__(NG * 64)
paged_decode_combine_kernel(const DecodeParams p, int T) {
  constexpr int F4ROW = D / 4;
  constexpr int PSTRIDE = D + 4;
  // Sequential path: up to CS partials, all in flight; CS <= NG keeps it
  // equal to the grouped definition.
  constexpr int CS = (32 / KCW) < NG ? 32 / KCW : NG;
  constexpr int CB = KCW >= 8 ? 1 : 8 / KCW;  // grouped path: partials in flight per wave
  __shared__ float s_m[NG][KCW * 64];
  __shared__ float s_l[NG][KCW * 64];
  __shared__ f32x4 s_o[NG][KCW * 64];
  __shared__ int s_cnt[NG], s_slot[NG];  // partial count and first slot of the tile's pieces

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int Hkv = p.num_kv_heads;
  const int G = p.num_q_heads / Hkv;
  const int Sq = p.q_len;
  const int nrows = G * Sq;
  const int f4_total = nrows * F4ROW;
  const int pieces = (f4_total + 64 * KCW - 1) / (64 * KCW);  // per unit
  const int64_t cstride = (int64_t)Hkv * nrows * PSTRIDE;     // floats between partial slots
  const int64_t npieces = (int64_t)p.num_seqs * Hkv * pieces;
  const int64_t v0 = (int64_t)blockIdx.x * T;
  const int tn = (int)min((int64_t)T, npieces - v0);

  // Piece v: unit u = v / pieces = (r, g); this lane's float4s f0 + 64 k.
  // A unit's float4s are numbered in the order pass 1 stores them: float4 f
  // of a partial slot holds dimensions (4 jg + i) NT + n0 .. + 3 of row rho,
  // where f = (k * 4 + jg) * nrows + rho and k = i NT / 4 + n0 / 4
  // (NT = D / 16); the (m, l) pairs of the rows follow the nrows * D floats.
  auto piece = [&](int64_t v, int& r, int& g, int& f0) {
    const int64_t u = v / pieces;
    f0 = (int)(v - u * pieces) * 64 * KCW + lane;
    r = (int)(u / Hkv);
    g = (int)(u - (int64_t)r * Hkv);
  };
  auto row_of = [&](int f) { return f % nrows; };
  auto ml_offset = [&](int f) { return nrows * D + 2 * row_of(f); };
  auto dim_of = [&](int f) {  // first dimension of float4 f
    constexpr int NT = D / 16;
    const int kj = f / nrows;  // k * 4 + jg
    const int k = kj >> 2, jg = kj & 3;
    const int i = k / (NT / 4), n0 = (k - i * (NT / 4)) * 4;
    return (4 * jg + i) * NT + n0;
  };
  auto partials_of = [&](int g, int slot) {
    return p.partials + ((int64_t)slot * Hkv + g) * nrows * PSTRIDE;
  };
  // Output float4 f of unit (r, g): normalise and store, with the row's lse.
  auto emit = [&](int r, int g, int f, float M, float Lt, f32x4 ot) {
    const int row = row_of(f);
    const int d = dim_of(f);
    const int jr = row / G;
    const int hr = row - jr * G;
    const float inv = Lt > 0.0f ? 1.0f / Lt : 0.0f;
    const int64_t orow = ((int64_t)r * Sq + jr) * (G * Hkv) + (int64_t)g * G + hr;
    *(f32x4*)(p.out + orow * D + d) = ot * inv;
    if (p.lse_out && d == 0) p.lse_out[orow] = row_lse(M, Lt);
  };

  // ---- wave w: piece w of the tile; merged here when 2 <= C <= CS ---------
  if (wave < tn) {
    int r, g, f0;
    piece(v0 + wave, r, g, f0);
    const int C = uniform(p.chunk_meta[2 * r + 1]);
    const int slot = uniform(p.chunk_meta[2 * r]);
    if (lane == 0) {
      s_cnt[wave] = C;
      s_slot[wave] = slot;
    }
    if (C >= 2 && C <= CS) {
      const float* base = partials_of(g, slot);
      f32x4 a[CS][KCW];
      f32x2 ml[CS][KCW];
#pragma unroll
      for (int j = 0; j < CS; ++j) {
#pragma unroll
        for (int k = 0; k < KCW; ++k) {
          const int f = f0 + 64 * k;
          if (j < C && f < f4_total) {
            a[j][k] = *(const f32x4*)(base + j * cstride + 4 * f);
            ml[j][k] = *(const f32x2*)(base + j * cstride + ml_offset(f));
          }
        }
      }
#pragma unroll
      for (int k = 0; k < KCW; ++k) {
        const int f = f0 + 64 * k;
        float M = -INFINITY, Lt = 0.0f;
        f32x4 ot = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < CS; ++j)
          if (j < C) merge_state(M, Lt, ot, ml[j][k][0], ml[j][k][1], a[j][k]);
        if (f < f4_total) emit(r, g, f, M, Lt, ot);
      }
    }
  }
  __syncthreads();

  // ---- pieces with C > CS, one after another: wave w merges group w --------
  for (int vi = 0; vi < tn; ++vi) {
    const int Cv = s_cnt[vi];
    if (Cv <= CS) continue;  // written by pass 1, or merged above
    int r, g, f0;
    piece(v0 + vi, r, g, f0);
    const float* base = partials_of(g, s_slot[vi]);
    float Mx[KCW], Ls[KCW];
    f32x4 o[KCW];
#pragma unroll
    for (int k = 0; k < KCW; ++k) {
      Mx[k] = -INFINITY;
      Ls[k] = 0.0f;
      o[k] = (f32x4){0.f, 0.f, 0.f, 0.f};
    }
    for (int c0 = wave; c0 < Cv; c0 += NG * CB) {
      f32x4 a[CB][KCW];
      f32x2 ml[CB][KCW];
#pragma unroll
      for (int j = 0; j < CB; ++j) {
        const int cc = c0 + j * NG;
#pragma unroll
        for (int k = 0; k < KCW; ++k) {
          const int f = f0 + 64 * k;
          if (cc < Cv && f < f4_total) {
            a[j][k] = *(const f32x4*)(base + (int64_t)cc * cstride + 4 * f);
            ml[j][k] = *(const f32x2*)(base + (int64_t)cc * cstride + ml_offset(f));
          }
        }
      }
#pragma unroll
      for (int j = 0; j < CB; ++j) {
#pragma unroll
        for (int k = 0; k < KCW; ++k)
          if (c0 + j * NG < Cv && f0 + 64 * k < f4_total)
            merge_state(Mx[k], Ls[k], o[k], ml[j][k][0], ml[j][k][1], a[j][k]);
      }
    }
#pragma unroll
    for (int k = 0; k < KCW; ++k) {
      s_m[wave][lane + 64 * k] = Mx[k];
      s_l[wave][lane + 64 * k] = Ls[k];
      s_o[wave][lane + 64 * k] = o[k];
    }
    __syncthreads();
    for (int i = threadIdx.x; i < 64 * KCW; i += NG * 64) {
      const int f = f0 - lane + i;  // float4 of the unit this thread combines
      if (f < f4_total) {
        float M = -INFINITY, Lt = 0.0f;
        f32x4 ot = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
        for (int w = 0; w < NG; ++w) merge_state(M, Lt, ot, s_m[w][i], s_l[w][i], s_o[w][i]);
        emit(r, g, f, M, Lt, ot);
      }
    }
    __syncthreads();
  }
}

// The merge of units made of `kc` columns of 64 float4s. One float4 per lane
// (pieces of one column) when all those pieces fit into one round of
// resident workgroups, or when requests average more than NG partials: the
// partials of a long context are then read by kc times as many compute
// units, with eight partials in flight per wave. Otherwise every lane takes
// 32 / NG float4s (one piece per unit), which keeps more loads in flight
// per wave. Tiles of
// T pieces, T the smallest count that fits one round (at most NG).
template <int D, int KCW, int NG>
hipError_t launch_merge_shape(const DecodeParams& p, int64_t n, int resident, hipStream_t stream) {
  int64_t T = (n + resident - 1) / resident;
  T = T < 1 ? 1 : (T > NG ? NG : T);
  const int64_t tiles = (n + T - 1) / T;  // <= 8192 requests x Hkv x 8 pieces
  paged_decode_combine_kernel<D, NG, KCW>
      <<<dim3((unsigned)tiles), dim3(NG * 64), 0, stream>>>(p, (int)T);
  return hipGetLastError();
}

template <int D, int NG>
hipError_t launch_merge(const DecodeParams& p, int kc, hipStream_t stream) {
  constexpr int KMAX = 32 / NG;  // float4s per lane that cover a unit of this NG
  static std::atomic<int> cache1[kMaxDevices], cachew[kMaxDevices];
  int res1 = 0, resw = 0;
  hipError_t e = resident_of(reinterpret_cast<const void*>(&paged_decode_combine_kernel<D, NG, 1>),
                             NG * 64, 0, cache1, &res1);
  if (e != hipSuccess) return e;
  const int64_t units = (int64_t)p.num_seqs * p.num_kv_heads;
  // One float4 per lane also when requests average more than NG partials:
  // at 32 / NG float4s per lane a wave of the grouped path keeps only
  // 8 / (32 / NG) partials in flight, and a long unit then waits on
  // several rounds of loads one after another.
  if (units * kc <= res1 || (int64_t)p.slices > (int64_t)NG * p.num_seqs)
    return launch_merge_shape<D, 1, NG>(p, units * kc, res1, stream);
  e = resident_of(reinterpret_cast<const void*>(&paged_decode_combine_kernel<D, NG, KMAX>),
                  NG * 64, 0, cachew, &resw);
  if (e != hipSuccess) return e;
  return launch_merge_shape<D, KMAX, NG>(p, units * ((kc + KMAX - 1) / KMAX), resw, stream);
}

// The split-K merge for the row count of these parameters.
template <int D>
hipError_t launch_merge_for(const DecodeParams& p, hipStream_t stream) {
  const int nrows = p.num_q_heads / p.num_kv_heads * p.q_len;
  const int kc = (nrows * (D / 4) + 63) / 64;
  if (kc <= 4) return launch_merge<D, merge_groups(4)>(p, kc, stream);
  return launch_merge<D, merge_groups(8)>(p, kc, stream);
}

}  // namespace

hipError_t decode_pass1_nc1(const DecodeParams& p, hipStream_t stream) {
  return pass1_for<1, 1>(p, stream);
}

hipError_t decode_slices_nc1(const DecodeParams& p, int* slices) { return slices_for<1, 1>(p, slices); }

int32_t decode_max_slices(int32_t num_kv_heads) {
  // Partial storage for up to 8192 waves' worth of slices (a 256-CU part
  // holds 2048 decode waves at once), so every resident slot gets a slice.
  const int32_t t = 8192 / (num_kv_heads > 0 ? num_kv_heads : 1);
  return t > 16 ? t : 16;
}

size_t decode_lds_bytes(int32_t num_seqs) {
  // pass 1's prefix of the requests' tiles (num_seqs + 1) and their lengths
  return (2 * (size_t)num_seqs + 1) * sizeof(int32_t);
}

size_t decode_meta_bytes(int32_t num_seqs) {
  return ((size_t)num_seqs * 2 * sizeof(int32_t) + 255) / 256 * 256;
}

size_t decode_partial_bytes(int32_t num_seqs, int32_t q_len, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t head_dim) {
  // Partial slot of (slice, request) is slice + request: every segment of
  // a slice's range has its own slot, below max_slices + num_seqs.
  return decode_partial_slot_bytes(q_len, num_q_heads, head_dim) *
         ((size_t)decode_max_slices(num_kv_heads) + (size_t)num_seqs);
}

size_t decode_partial_slot_bytes(int32_t q_len, int32_t num_q_heads, int32_t head_dim) {
  return (size_t)num_q_heads * (size_t)q_len * (size_t)(head_dim + 4) * sizeof(float);
}

// Column tiles of 16 query rows per wave for the rows of one KV head.
static int decode_column_tiles(const DecodeParams& p) {
  const int nrows = p.num_q_heads / p.num_kv_heads * p.q_len;
  return nrows <= 16 ? 1 : nrows <= 32 ? 2 : 4;
}

hipError_t decode_slices(const DecodeParams& p, int* slices) {
  switch (decode_column_tiles(p)) {
    case 1: return decode_slices_nc1(p, slices);
    case 2: return decode_slices_nc2(p, slices);
    default: return decode_slices_nc4(p, slices);
  }
}

hipError_t launch_paged_decode(const DecodeParams& pin, hipStream_t stream) {
  DecodeParams p = pin;
  hipError_t e = decode_slices(p, &p.slices);
  if (e != hipSuccess) return e;
  switch (decode_column_tiles(p)) {
    case 1: e = decode_pass1_nc1(p, stream); break;
    case 2: e = decode_pass1_nc2(p, stream); break;
    default: e = decode_pass1_nc4(p, stream); break;
  }
  if (e != hipSuccess) return e;
  if (p.head_dim == 128) return launch_merge_for<128>(p, stream);
  return launch_merge_for<64>(p, stream);
}

}  // namespace kvs
