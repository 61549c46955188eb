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
// A sliding-window layer ("KV Caching with vLLM", section "Attention Type";
// "Decode Context-Length Bucketing", the SWA tail trim) adds two things: a
// window, so the query at qpos sees keys from qpos - window + 1 only, and a
// per-request kv_pos_offset, the absolute position of the (tail-trimmed)
// table's column 0; positions stay absolute.
//
// How, on CDNA4:
// * Work split: the 16-token tiles of every request's context, laid end to
//   end over the batch, are cut into `slices` equal ranges, one per
//   resident workgroup slot (eight waves per compute unit; four for the fp32
//   kernels of four KV heads per workgroup), so every
//   workgroup streams the same number of bytes and all finish together (no
//   rounds, no tail of short units). A
//   range may start or end inside a request and may span requests; each
//   (slice, request) piece is a segment. A workgroup holds the waves of NW
//   KV heads (their [block][token][head] rows are adjacent in HBM); a head
//   has one wave, or (up to 16 query rows, bf16) WS waves that split its
//   tiles round robin by absolute tile index, each with a softmax state of
//   its own, pooled through LDS and merged in wave order at the segment's
//   end. Two heads of four waves each stream faster than eight heads of one
//   (the workgroup has four tiles in flight per head instead of one) and cut
//   the batch into a quarter as many slices, so fewer partial states.
// * The cut is made on the device from seq_lens (no host synchronisation):
//   every workgroup scans the batch's tile counts into an LDS prefix. It
//   depends only on the visible context lengths and the device, so a
//   head-trimmed walk, a full-table walk and the context walk produce the
//   same partials.
// * The block ids of a segment are staged in LDS by the workgroup (pieces of
//   up to 256 blocks), so each tile's block id is an LDS read that does not
//   hold up the vector-memory pipeline.
// * The tile loop is straight-line: the loads of tile t+1 are issued before
//   tile t is computed and are never under a data-dependent branch (an
//   inactive table entry reads null block 0 and is masked; the loop tail
//   re-loads its last tile, which hits in cache), so one tile stays in
//   flight behind the one being computed. A bare barrier every tile step
//   keeps the waves of a workgroup in step (every two steps with two row
//   groups per head); it waits for no load in flight, where __syncthreads()
//   would wait for all of them.
// * Tile of 16 tokens. The query rows of a KV head ((query token, head in
//   group) pairs, up to 64) form column tiles of 16: NC of them per wave, and
//   above 32 rows two row groups per KV head share the rows. Both need every
//   tile and each wave loads it, the second read hitting in cache (V then
//   without the nontemporal hint, so that its lines stay for the partner).
//   (Sharing one LDS ring, each wave loading half of the tile, was slower:
//   each step's barrier then waits for both halves to land.) S^T = K Q^T on
//   v_mfma_f32_16x16x32_bf16 (fp32 KV: v_mfma_f32_16x16x4f32), once per
//   column tile: K is the A operand (lane l holds token l % 16, 16 bytes of
//   its head row per piece), Q^T the B operand (lane l holds query row
//   16 c + l % 16). The result gives each lane four tokens of one row.
//   bf16 K does not load in that layout (each instruction would read a
//   64-byte piece of sixteen rows 2 KB apart):
//   direct-to-LDS loads read whole head rows into a per-wave LDS ring,
//   stored with the chunk index XORed by the token, and each lane reads its
//   operand pieces back (conflict-free) just before the score MFMA.
// * Online softmax per query row, in exp2 units, with a lazily moved
//   exponent reference (at most 8 below the running max), entirely inside the lane
//   except one max over the four lane groups (two permlane swaps).
// * O^T = V^T P^T, per column tile. Lane l reads a 16-byte slice of the
//   head rows of tokens 4 * (l / 16) .. + 3 (each 16-lane group reads whole
//   256-byte head rows: V stays in its natural layout), and dimension column
//   l % 16 of n-tile n is dimension (l % 16) * NT + n. bf16 KV: two
//   v_mfma_f32_16x16x32_bf16 per n-tile take the 16 tokens at once, the A
//   operand packed from those slices with v_perm (each token's value twice
//   along the contraction), the B operand P^T in bf16: P is split exactly
//   into three bf16 terms (each the truncation of what the previous left),
//   (hi, mid) in the first and (lo, 0) in the second, so the products equal
//   those of fp32 P. fp32 KV:
//   v_mfma_f32_16x16x4f32, four tokens per step. The accumulator lands with
//   query row 16 c + l % 16, matching the softmax state.
// * A segment that holds a whole request writes its output. Otherwise its
//   partial state (acc, m, l per row) goes to slot slice + request of the
//   workspace, and a second kernel merges a request's partials in one fixed
//   association (below), so results do not depend on scheduling, on the
//   launch shape or on the batch around the request.
// * Masked keys are removed by select, never by multiplying by zero, and the
//   values of keys past the context are replaced by -0.0, so unwritten (NaN
//   canary) cache rows cannot leak into the output and a masked product is
//   -0.0, which leaves every accumulator bit-unchanged.
// * The fixed-shape table walk is a separate instantiation: it computes
//   the same segments, then reads every walked column past each context
//   (cut the same way over the slices) and folds those bytes into a sink
//   that is stored only under a flag the host never sets.
#pragma once

#include <math.h>

#include <atomic>
#include <type_traits>

#include "kvslot_internal.h"
#include "slot_formula.h"

namespace kvs {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr uint32_t kFlagWalkTable = 0x1u;
// Never set by the host. Testing it keeps the table-walk loads alive.
constexpr uint32_t kFlagSink = 0x80000000u;
// pass-1 modes: context walk, fixed-shape table walk, the general walk
// (sliding window, tail-trimmed table, context-parallel share), and the
// context walk that first writes the step's new tokens (append)
constexpr int kContextWalk = 0, kTableWalk = 1, kGeneral = 2, kAppend = 3;
constexpr int kTile = 16;
constexpr int kStage = 256;  // block ids staged in LDS at a time
constexpr int kDepth = 2;    // tiles in flight per wave

// s_waitcnt immediates (gfx9 encoding): wait until at most n vector memory
// operations of this wave are outstanding; lgkmcnt and expcnt not waited on.
constexpr int vmcnt_imm(int n) { return (n & 0xf) | ((n >> 4) << 14) | (0x7 << 4) | (0xf << 8); }
constexpr int kVmcnt0 = vmcnt_imm(0);

// Wavefront scans on DPP: four row shifts build the prefix inside each row
// of 16 lanes, two row broadcasts carry it across rows. Values move lane to
// lane in the VALU, with no LDS round trip. Every lane must be active.
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_add(int x) {
  return x + __builtin_amdgcn_update_dpp(0, x, CTRL, ROWS, 0xf, false);
}

__device__ __forceinline__ int wave_inclusive_scan(int x) {
  x = dpp_add<0x111, 0xf>(x);  // row_shr:1
  x = dpp_add<0x112, 0xf>(x);  // row_shr:2
  x = dpp_add<0x114, 0xf>(x);  // row_shr:4
  x = dpp_add<0x118, 0xf>(x);  // row_shr:8
  x = dpp_add<0x142, 0xa>(x);  // row_bcast:15 into rows 1 and 3
  x = dpp_add<0x143, 0xc>(x);  // row_bcast:31 into rows 2 and 3
  return x;
}


// Reductions over the four 16-lane groups of a wavefront (lanes l, l ^ 16,
// l ^ 32, l ^ 48): permlane16_swap pairs rows 0-1 and 2-3, permlane32_swap
// pairs the two halves. Each lane receives its partner's value; both
// operands of the combine are then the same in every lane of the group.
__device__ __forceinline__ float max_over_groups(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float sum_over_groups(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// The tiles request r walks: absolute positions [16 * t_lo, E) in 16-token
// tiles, n of them. off is the absolute position of table column 0 (a
// tail-trimmed table; 0 for a whole table), rounded down to a block. E ends
// the visible context: the request's length, cut at the walked columns. With
// a sliding window the walk starts at the earliest key a query of this step
// sees (L - q_len - window + 1). Positions stay below 2^31 - 64.
struct ReqSpan {
  int off, E, t_lo, n;
};

// Under context parallelism the walk runs over this rank's own positions
// (its cache's local positions, 0 .. E - 1): the global positions below
// min(L, walk_blocks * world * bs) that this rank stores.
template <bool GEN>
__device__ __forceinline__ ReqSpan request_span(const DecodeParams& p, int r, int L, int walk_tok,
                                                int bs, int Sq) {
  ReqSpan sp;
  if (GEN && p.cp_world > 1) {
    const int64_t eg = min((int64_t)L, (int64_t)walk_tok * p.cp_world);
    const int64_t run = (int64_t)1 << p.cp_ishift;
    const int64_t span = run * p.cp_world;
    const int64_t rem = eg > 0 ? eg % span - (int64_t)p.cp_rank * run : 0;
    const int64_t e_loc = eg > 0 ? (eg / span) * run + min(max(rem, (int64_t)0), run) : 0;
    sp.off = 0;
    sp.E = (int)min(e_loc, (int64_t)INT32_MAX - 64);
    sp.t_lo = 0;
    sp.n = (sp.E + 15) / 16;
    return sp;
  }
  const int32_t* kv_pos_offset = p.kv_pos_offset;
  const int32_t window = p.window;
  const int off = GEN && kv_pos_offset ? kv_pos_offset[r] : 0;
  sp.off = max(off, 0) & ~(bs - 1);
  int64_t E = min((int64_t)L, (int64_t)sp.off + walk_tok);
  E = min(E, (int64_t)INT32_MAX - 64);
  sp.E = L <= 0 ? 0 : (int)E;
  int64_t start = sp.off;
  if (GEN && window > 0) start = max(start, (int64_t)L - Sq - window + 1);
  sp.t_lo = (int)(start / 16);
  sp.n = sp.E > start ? (sp.E + 15) / 16 - sp.t_lo : 0;
  return sp;
}

// Natural-log sum of exp(scores) of a row from its running state: max m
// (log2 units) and sum l of exp2(score - m); -inf when the row saw no key.
__device__ __forceinline__ float row_lse(float m, float l) {
  return l > 0.0f ? (m + log2f(l)) * 0.69314718055994531f : -INFINITY;
}

// v_perm_b32 selectors over {x (bytes 4-7), y (bytes 0-3)}: the low halves
// of y and x, or their high halves, as one pair (y's half first).
constexpr uint32_t kPermLo = 0x05040100u, kPermHi = 0x07060302u;

// The high 16 bits of two floats (their bf16 truncations), a first: one
// bf16 pair.
__device__ __forceinline__ uint32_t bf16_pair_hi(float a, float b) {
  return __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), kPermHi);
}

// MODE: kContextWalk, kTableWalk (the fixed-shape walk) or kGeneral (a
// sliding window over a possibly tail-trimmed table, or one rank's share
// under context parallelism).
// NC: column tiles of 16 query rows per wave; RH: row groups per KV head,
// each holding 16 NC consecutive rows of the head's (Hq / Hkv) * q_len rows
// (at most 16 NC RH). The row groups of one head need the same K and V tiles:
// each reads the whole tile, the second read hitting in cache. WS: waves that split the tiles of a head
// (and row group): wave s
// takes the tiles whose absolute index is s mod WS, keeping its own softmax
// state for its rows; at the end of a segment the WS states are pooled in LDS
// and merged in wave order. Waves of a workgroup: NW KV heads times RH times
// WS, the head fastest.
template <bool BF16, int D, int NW, int MODE, int NC, int RH, int WS>
__global__ void __launch_bounds__(NW * RH * WS * 64, 2)
paged_decode_kernel(const DecodeParams p, int bs_shift) {
  constexpr int ES = BF16 ? 2 : 4;       // bytes per element
  constexpr int EP = 16 / ES;            // elements per 16-byte piece
  constexpr int NP = D / (4 * EP);       // 16-byte K pieces per lane per token
  constexpr int NT = D / 16;             // P.V n-tiles (dimension columns of 16)
  constexpr int NVW = NT * ES / 4;       // V dwords per lane per token
  constexpr int PSTRIDE = D + 4;         // floats per partial row (acc, m, l, pad)
  constexpr int NTHR = NW * RH * WS * 64;
  constexpr int NWAVES = NW * RH * WS;
  constexpr bool TW = MODE == kTableWalk;
  constexpr bool GEN = MODE == kGeneral;
  constexpr bool APP = MODE == kAppend;
  constexpr uint32_t kNegZero = BF16 ? 0x80008000u : 0x80000000u;
  static_assert(NP >= 1 && NVW >= 2, "unsupported head_dim");
  static_assert(WS == 1 || WS == 2 || WS == 4 || WS == 8, "WS: a power of two up to 8");
  struct TileBuf {
    u32x4 k[NP];         // K pieces of token rho of the tile
    uint32_t v[4][NVW];  // V slices of tokens 4*jg .. 4*jg+3
    int bid;             // block id the tile was read from (0: inactive entry)
  };
  constexpr int DEPTH = kDepth;
  using RingBuf = TileBuf;
  // [num_seqs + 1]: first tile of each request; then [num_seqs]: its length
  extern __shared__ int s_pref[];
  int* const s_len = s_pref + p.num_seqs + 1;
  __shared__ int s_blk[kStage];
  __shared__ int s_wave[NWAVES], s_wave_n[NWAVES];
  // append: the step tokens whose rows this slice reads, and their slots
  __shared__ int s_app_t[APP ? NTHR : 1];
  __shared__ int64_t s_app_s[APP ? NTHR : 1];
  __shared__ int s_app_n;
  // request holding this slice's first unit (context), first padding tile,
  // and the context tiles of the requests before the latter
  __shared__ int s_first[3];
  // the tile split's pool: every wave's state of one column tile at a
  // segment's end, per lane
  constexpr int NPOOL = WS > 1 ? NWAVES * 64 : 1;
  // bf16 K reaches the MFMA through LDS: each tile's K is read as whole head
  // rows by direct-to-LDS loads into a ring of DEPTH slots per wave (V stays
  // in registers), which shares its LDS with the pool (a segment's walk and
  // its pooling never overlap). A head row is CH 16-byte chunks; one load
  // instruction covers TPI whole rows, NI of them a tile. Chunk c of token t
  // sits at 16-byte slot CH t + (c ^ (t mod CH)) of its slot: the XOR keeps
  // the operand reads below free of bank conflicts.
  constexpr bool KL = BF16;
  constexpr int CH = D * ES / 16;
  constexpr int TPI = 64 / CH;
  constexpr int NI = kTile / TPI;
  constexpr int KSLOT = kTile * CH;  // f32x4 per tile's K
  constexpr int NRING = KL ? NWAVES * DEPTH * KSLOT : 1;
  constexpr int NPL = WS > 1 ? NPOOL * NT : 1;
  constexpr int NBIG = NPL > NRING ? NPL : NRING;
  __shared__ f32x4 s_pool[NBIG];
  __shared__ float s_pm[NPOOL], s_pl[NPOOL];

  const int lane = threadIdx.x & 63;
  // wave-uniform (in a scalar register): the wave's head, rows, tile share and
  // every tile's address base follow from it without per-lane arithmetic
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int rho = lane & 15;  // query row owned by this lane (MFMA column)
  const int jg = lane >> 4;   // lane group: tokens 4*jg .. 4*jg+3 of a tile

  const int B = p.num_seqs;
  const int bs = 1 << bs_shift;
  const int walk_tok = p.walk_blocks << bs_shift;
  const int walk_tiles = walk_tok / kTile;
  const int Hkv = p.num_kv_heads;
  const int Hq = p.num_q_heads;
  const int G = Hq / Hkv;
  const int Sq = p.q_len;
  const int nrows = G * Sq;
  const int HG = Hkv / NW;  // the launcher picks NW dividing Hkv
  const int S = p.slices;
  const int slice = blockIdx.x / HG;
  const int hg = blockIdx.x - slice * HG;
  const int g = hg * NW + wave % NW;  // this wave's KV head
  // waves: head in group fastest, then row group, then tile share
  const int rh = RH > 1 ? (wave / NW) % RH : 0;
  const int row0 = 16 * NC * rh;                // its first query row of that head
  const int ws = WS > 1 ? wave / (NW * RH) : 0;  // its share of the head's tiles
  const int64_t block_bytes = ((int64_t)Hkv * D * ES) << bs_shift;
  const uint32_t row_bytes = (uint32_t)(Hkv * D * ES);

  // ---- work prefix of the batch, in LDS ------------------------------------
  // The context tiles of all requests, laid end to end, are cut into S equal
  // ranges, one per slice; a slice's range may start or end inside a
  // request and may cover several requests. Its pieces are the segments.
  // Each request with context also counts X units ahead of its
  // tiles (the cost of starting a segment), so a slice that starts a
  // request carries that many fewer tiles. s_pref holds these units.
  // (start_tiles is the cost in steps of a wave; a workgroup whose waves split
  // each head's tiles takes WS tiles per step)
  const int X = p.start_tiles * WS;
  // The first request of this thread's share is loaded here, before the
  // append's token loads, so that waiting for it does not wait for them.
  const int len0 = (int)threadIdx.x < B ? p.seq_lens[threadIdx.x] : 0;
  // append: this thread's step token and its slot, looked up before the
  // scan below so that the table read overlaps it
  // (the slot formula of slot_formula.h, with its table read issued here and
  // its value first used after the scan)
  int app_r = -1, app_blk = 0;
  int64_t app_p = -1, app_lb = -1;
  if constexpr (APP) {
    if ((int64_t)threadIdx.x < p.app_tokens) {
      app_r = p.app_req[threadIdx.x];
      app_p = p.app_pos[threadIdx.x];
    }
  }
  if ((int)threadIdx.x < B) {
    s_pref[threadIdx.x] = request_span<GEN>(p, threadIdx.x, len0, walk_tok, bs, Sq).n;
    s_len[threadIdx.x] = len0;
  }
  if constexpr (APP) {
    if (app_r >= 0 && app_r < B && app_p >= 0 && (app_p >> bs_shift) < p.table_stride) {
      app_lb = app_p >> bs_shift;
      app_blk = p.block_table[(int64_t)app_r * p.table_stride + app_lb];
    }
  }
  for (int rr = threadIdx.x + NTHR; rr < B; rr += NTHR) {
    const int len = p.seq_lens[rr];
    s_pref[rr] = request_span<GEN>(p, rr, len, walk_tok, bs, Sq).n;
    s_len[rr] = len;
  }
  if (threadIdx.x == 0) {
    s_first[0] = 0;
    s_first[1] = 0;
    s_first[2] = 0;
  }
  __syncthreads();
  const int per = (B + NTHR - 1) / NTHR;  // contiguous requests per thread
  const int rb = min((int)threadIdx.x * per, B);
  const int re = min(rb + per, B);
  int local = 0, local_n = 0;  // units and tiles of this thread's requests
  for (int rr = rb; rr < re; ++rr) {
    const int n = s_pref[rr];
    local += n > 0 ? n + X : 0;
    local_n += n;
  }
  const int incl = wave_inclusive_scan(local);
  const int incl_n = TW ? wave_inclusive_scan(local_n) : 0;
  if (lane == 63) {
    s_wave[wave] = incl;
    s_wave_n[wave] = incl_n;
  }
  __syncthreads();
  int total = 0, run = incl - local, total_n = 0, run_n = incl_n - local_n;
#pragma unroll
  for (int w = 0; w < NWAVES; ++w) {
    const int t = s_wave[w];
    const int tn = s_wave_n[w];
    total += t;
    run += w < wave ? t : 0;
    total_n += tn;
    run_n += w < wave ? tn : 0;
  }
  // total <= num_seqs * (walk_tiles + X) < 2^31 (checked by the host)
  const int Q = max((total + S - 1) / S, p.min_tiles);  // units per slice
  const int a = (int)min((int64_t)slice * Q, (int64_t)total);
  const int b = (int)min((int64_t)a + Q, (int64_t)total);
  // Fixed-shape walk: the columns past each request's context (its padding
  // tiles) are cut evenly into a second range per slice.
  const int pad_total = TW ? B * walk_tiles - total_n : 0;
  const int Qp = max((pad_total + S - 1) / S, p.min_tiles);
  const int pa = (int)min((int64_t)slice * Qp, (int64_t)pad_total);
  const int pbnd = (int)min((int64_t)pa + Qp, (int64_t)pad_total);
  for (int rr = rb; rr < re; ++rr) {
    const int n = s_pref[rr];
    const int wu = n > 0 ? n + X : 0;
    if (run <= a && a < run + wu) s_first[0] = rr;
    if (TW) {
      const int pr = rr * walk_tiles - run_n;  // padding tiles before request rr
      if (pr <= pa && pa < pr + (walk_tiles - n)) {
        s_first[1] = rr;
        s_first[2] = run_n;
      }
    }
    s_pref[rr] = run;
    run += wu;
    run_n += n;
  }
  if (threadIdx.x == 0) s_pref[B] = total;
  if constexpr (APP) {
    if (threadIdx.x == 0) s_app_n = 0;
  }
  __syncthreads();

  // ---- append: write the step's new K/V rows before any tile is read ------
  // A row lies in one tile of its request; the slice holding that tile (the
  // cut above) writes it, each head's first wave its own KV head's part, so
  // the wave that later loads those bytes is the one that stored them, and it
  // waits for its stores before going on (with two waves per head, the other
  // one waits at a workgroup barrier). Rows of positions no slice reads (past
  // the walked tiles) and the slot mapping itself are written by workgroup 0.
  if constexpr (APP) {
    constexpr int PR = D * ES / 16;  // 16-byte pieces of one head's row
    const int64_t T = p.app_tokens;
    const int64_t total_slots = p.total_blocks << bs_shift;
    const bool first_wg = blockIdx.x == 0;
    int owner = -1;  // slice that reads this token's tile
    if (app_r >= 0 && app_r < B && app_p >= 0) {
      const int wu = s_pref[app_r + 1] - s_pref[app_r];
      const int64_t k = app_p >> 4;
      if (wu > 0 && k < wu - X) owner = (s_pref[app_r] + X + (int)k) / Q;
    }
    const bool own = owner == slice;
    const int64_t s =
        app_lb >= 0 && app_blk > 0 ? (int64_t)app_blk * bs + (app_p - (app_lb << bs_shift)) : -1;
    const bool inb = s >= 0 && s < total_slots;
    if (first_wg && (int64_t)threadIdx.x < p.app_max_tokens)
      p.app_slots[threadIdx.x] = (int64_t)threadIdx.x < T ? s : -1;
    const u32x4* kn = (const u32x4*)p.app_k;
    const u32x4* vn = (const u32x4*)p.app_v;
    u32x4* kc = (u32x4*)p.app_k_cache;
    u32x4* vc = (u32x4*)p.app_v_cache;
    if (first_wg && (int64_t)threadIdx.x < T && inb && owner < 0) {
      for (int q4 = 0; q4 < Hkv * PR; ++q4) {
        kc[s * Hkv * PR + q4] = kn[(int64_t)threadIdx.x * Hkv * PR + q4];
        vc[s * Hkv * PR + q4] = vn[(int64_t)threadIdx.x * Hkv * PR + q4];
      }
    }
    if (own && inb) {
      const int i = atomicAdd(&s_app_n, 1);
      s_app_t[i] = (int)threadIdx.x;
      s_app_s[i] = s;
    }
    __syncthreads();
    const int n_own = s_app_n;
    for (int k0 = 0; k0 < n_own && wave < NW; k0 += 64 / PR) {
      const int kk = k0 + lane / PR;
      if (kk < n_own) {
        const int pc = lane % PR;
        const int64_t src = ((int64_t)s_app_t[kk] * Hkv + g) * PR + pc;
        const int64_t dst = (s_app_s[kk] * Hkv + g) * PR + pc;
        kc[dst] = kn[src];
        vc[dst] = vn[src];
      }
    }
    if (n_own > 0) __builtin_amdgcn_s_waitcnt(0);  // this wave's stores land before its loads
    if constexpr (RH > 1 || WS > 1) {
      if (n_own > 0) __syncthreads();  // and before the other waves of its head load them
    }
  }

  uint32_t sink = 0;
  const uint32_t k_lane_off = ((uint32_t)rho * Hkv + g) * (D * ES) + jg * 16;
  const uint32_t v_lane_off = ((uint32_t)(4 * jg) * Hkv + g) * (D * ES) + rho * (NT * ES);
  // K through LDS: this lane's byte offset in the tile for load instruction
  // i (token TPI i + lane / CH, chunk (lane mod CH) ^ token), and its byte
  // offset in a ring slot for operand piece pp (token rho, chunk 4 pp + jg,
  // the chunk the query's piece pp holds in this lane).
  uint32_t k_dma_off[KL ? NI : 1];
  int k_rd[KL ? NP : 1];
  if constexpr (KL) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int t = TPI * i + lane / CH;
      const int c = (lane % CH) ^ (t % CH);
      k_dma_off[i] = (uint32_t)t * row_bytes + (uint32_t)g * (D * ES) + 16u * (uint32_t)c;
    }
#pragma unroll
    for (int pp = 0; pp < NP; ++pp)
      k_rd[pp] = (int)(16 * ((uint32_t)(CH * rho + ((4 * pp + jg) ^ (rho % CH)))));
  }
  // The operand pieces of the tile in ring slot `base` (an f32x4 index),
  // read in one asm block that also waits for them: the compiler then adds no
  // wait of its own for the direct-to-LDS loads in flight to the other slot.
  // The outputs are early-clobber: a read's destination must not be the
  // address register of a later read in the block (its data may land first).
  auto read_k_slot = [&](u32x4 (&k)[NP], int base) {
    const uint32_t a = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) f32x4*)
                           (&s_pool[base]);
    if constexpr (NP == 4) {
      asm volatile(
          "ds_read_b128 %0, %4\n\t"
          "ds_read_b128 %1, %5\n\t"
          "ds_read_b128 %2, %6\n\t"
          "ds_read_b128 %3, %7\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3])
          : "v"(a + k_rd[0]), "v"(a + k_rd[1]), "v"(a + k_rd[2]), "v"(a + k_rd[3])
          : "memory");
    } else {
      static_assert(!KL || NP == 2, "head_dim 64 or 128");
      asm volatile(
          "ds_read_b128 %0, %2\n\t"
          "ds_read_b128 %1, %3\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(k[0]), "=&v"(k[1])
          : "v"(a + k_rd[0]), "v"(a + k_rd[1])
          : "memory");
    }
  };
  // Tiles [tok_a, tok_b) (absolute positions, multiples of kTile) of table
  // row trow, whose column 0 holds position off, through fn(position of the
  // tile, its loads). Block ids are staged in LDS in pieces
  // of kStage; a ring of kDepth tile buffers keeps tiles t+1 .. t+kDepth-1
  // in flight while tile t is used. Loads past the last tile re-load the
  // last tile (a cache hit), so no load depends on a branch.
  auto walk_tiles_of = [&](const int32_t* trow, int off, int tok_a, int tok_b, auto&& fn,
                           auto&& after_first_prologue) {
    const int blk_first = (tok_a - off) >> bs_shift;
    const int blk_end = ((tok_b - 1 - off) >> bs_shift) + 1;
    for (int pb = blk_first; pb < blk_end; pb += kStage) {
      const int pn = min(kStage, blk_end - pb);
      // K through LDS: the previous piece's last loads into the ring land
      // before this piece's first ones are issued
      if constexpr (KL) __builtin_amdgcn_s_waitcnt(kVmcnt0);
      __syncthreads();  // the previous piece (and segment's pooled states) is consumed
      for (int i = threadIdx.x; i < pn; i += NTHR) {
        const int col = pb + i;
        s_blk[i] = col < p.table_stride ? trow[col] : 0;
      }
      __syncthreads();
      const int t_begin = max(tok_a, off + (pb << bs_shift));
      const int t_end = min(tok_b, off + ((pb + pn) << bs_shift));
      const int nt = (t_end - t_begin) / kTile;

      // K as the score MFMA's A operand, V in row layout. An inactive
      // entry reads null block 0 and is masked by the caller. V rows are
      // read with the nontemporal hint (streamed past the caches): on
      // MI355X that lifts long streams of reads from ~6.4 to ~7 TB/s; with
      // two row groups per head, whose second read of each tile must hit in
      // cache, they are plain loads. bf16 K goes to ring slot sl in LDS as
      // whole head rows (each load instruction reads TPI complete 256-byte
      // rows: about 7.1 TB/s for the K and V stream, against 6.7 TB/s when
      // every instruction reads a 64-byte piece of sixteen rows, the operand
      // layout in registers); fp32 K is a plain load into registers.
      // A load past the last tile (`tail`) re-loads the last tile and is never
      // used; its V part then reads the same rows of the K cache, lines the
      // tile's K loads just brought in, instead of missing again on V (whose
      // nontemporal loads are not kept in cache).
      auto load = [&](int tt, RingBuf& bf, int sl, bool tail) {
        const int bid = uniform(s_blk[((tt - off) >> bs_shift) - pb]);
        const bool active = bid > 0 && (int64_t)bid < p.total_blocks;
        const int64_t base = (int64_t)(active ? bid : 0) * block_bytes;
        const char* kb = (const char*)p.k_cache + base;
        const char* vb = (const char*)(tail ? p.k_cache : p.v_cache) + base;
        const uint32_t in_blk = (uint32_t)(tt & (bs - 1)) * row_bytes;
        bf.bid = active ? bid : 0;
        if constexpr (KL) {
          f32x4* slot = &s_pool[(wave * DEPTH + sl) * KSLOT];
          asm volatile("" ::: "memory");  // after the slot's last operand reads
#pragma unroll
          for (int i = 0; i < NI; ++i)
            __builtin_amdgcn_global_load_lds(
                (const void*)(kb + in_blk + k_dma_off[i]),
                (__attribute__((address_space(3))) void*)(slot + i * 64), 16, 0, 0);
        } else {
#pragma unroll
          for (int pp = 0; pp < NP; ++pp)
            bf.k[pp] = *(const u32x4*)(kb + in_blk + k_lane_off + pp * 64);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const char* src = vb + in_blk + v_lane_off + i * row_bytes;
          if constexpr (NVW == 2) {
            const u32x2 x = RH == 1 ? __builtin_nontemporal_load((const u32x2*)src)
                                    : *(const u32x2*)src;
            bf.v[i][0] = x[0];
            bf.v[i][1] = x[1];
          } else {
#pragma unroll
            for (int w = 0; w < NVW; w += 4) {
              const u32x4 x = RH == 1 ? __builtin_nontemporal_load((const u32x4*)(src + w * 4))
                                      : *(const u32x4*)(src + w * 4);
              bf.v[i][w] = x[0];
              bf.v[i][w + 1] = x[1];
              bf.v[i][w + 2] = x[2];
              bf.v[i][w + 3] = x[3];
            }
          }
        }
      };
      // This wave's tiles of the piece: those whose absolute tile index is ws
      // mod WS (all of them when WS = 1), t_first, t_first + WS, ..., nw of
      // them. Every wave of the workgroup runs the same number of steps (the
      // barrier below), loading past its last tile (or the piece's first tile
      // when it has none) where it has no tile.
      const int t_first = WS > 1 ? (ws - (t_begin >> 4)) & (WS - 1) : 0;
      const int nw = WS > 1 ? (nt > t_first ? (nt - t_first + WS - 1) / WS : 0) : nt;
      const int steps = WS > 1 ? (nt + WS - 1) / WS : nt;
      auto tile_at = [&](int u) {
        return t_begin + (nw > 0 ? t_first + min(u, nw - 1) * WS : 0) * kTile;
      };
      RingBuf bufs[DEPTH];
#pragma unroll
      for (int s = 0; s < DEPTH - 1; ++s) load(tile_at(s), bufs[s], s, s >= nw);
      if (pb == blk_first) after_first_prologue();
      for (int t = 0; t < steps; t += DEPTH) {
#pragma unroll
        for (int s = 0; s < DEPTH; ++s) {
          // Keep the workgroup's waves in step (they walk the same tiles, or
          // the same tiles' neighbours): every step, or every kDepth steps
          // with two row groups per head (each measured the faster there). Two
          // waves share each SIMD, and the older one wins issue arbitration;
          // left alone it runs ahead and the other finishes its last tiles
          // with half the loads in flight. A bare s_barrier waits for no
          // memory access, so the tiles already requested stay in flight
          // across it.
          if (RH == 1 || s == 0) __builtin_amdgcn_s_barrier();
          load(tile_at(t + s + DEPTH - 1), bufs[(s + DEPTH - 1) % DEPTH], (s + DEPTH - 1) % DEPTH,
               t + s + DEPTH - 1 >= nw);
          if constexpr (KL) {
            // Tile t + s is in (its K in slot s) once at most the loads just
            // issued (one tile's: NI to LDS, four V) are outstanding. Waited
            // for at every step, with a tile or not, so that the compiler
            // finds the older loads done on every path and adds no wait of
            // its own. The empty asm statements keep it from moving memory
            // accesses across the wait.
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(NI + 4));
            asm volatile("" ::: "memory");
          }
          if (t + s < nw) {
            if constexpr (KL) read_k_slot(bufs[s].k, (wave * DEPTH + s) * KSLOT);
            fn(t_begin + (t_first + (t + s) * WS) * kTile, bufs[s]);
          }
        }
      }
    }
  };

  // ---- one segment: tiles [t0, t1) of request r (nr tiles, tile 0 at unit pr) --
  auto segment = [&](int r, int t0, int t1, int nr, int pr) {
    const int L = uniform(s_len[r]);  // from LDS: no memory round trip at a segment start
    const ReqSpan sp = request_span<GEN>(p, r, L, walk_tok, bs, Sq);
    const int E = uniform(sp.E);
    const int off = uniform(sp.off);
    const int t_lo = uniform(sp.t_lo);

    // Query rows 16 c + rho, c < NC (rows are (query token, head in group));
    // the B operand of the score MFMA of column tile c.
    const int qpos_min = L - Sq;
    const int all_lo =
        GEN && p.window > 0 ? (int)max((int64_t)L - p.window, (int64_t)INT32_MIN) : INT32_MIN;
    int jrow[NC], hh[NC], qpos[NC], qlo[NC];
    u32x4 qp[NC][NP];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int row = row0 + 16 * c + rho;
      jrow[c] = row / G;
      hh[c] = row - jrow[c] * G;
      qpos[c] = row < nrows ? L - Sq + jrow[c] : -1;
      // sliding window: the row sees keys from qpos - window + 1; every row
      // does from L - window on
      qlo[c] = GEN && p.window > 0
                   ? (int)max((int64_t)qpos[c] - p.window + 1, (int64_t)INT32_MIN)
                   : INT32_MIN;
    }
    // The query pieces, loaded once the segment's first tiles are requested
    // (walk_tiles_of calls this after its first prologue), so that their round
    // trip overlaps the tiles' instead of preceding the table staging.
    auto load_q = [&]() {
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int row = row0 + 16 * c + rho;
        const char* qrow = (const char*)p.q +
                           ((((int64_t)r * Sq + jrow[c]) * Hq + (int64_t)g * G + hh[c]) * D) * ES;
#pragma unroll
        for (int pp = 0; pp < NP; ++pp) {
          qp[c][pp] = (u32x4){0u, 0u, 0u, 0u};
          if (row < nrows) qp[c][pp] = *(const u32x4*)(qrow + pp * 64 + jg * 16);
        }
      }
    };
    // Global position of a walked position: itself, except under context
    // parallelism, where the walk runs over this rank's local positions.
    auto gpos = [&](int lp) -> int64_t {
      if constexpr (GEN) {
        const int64_t run = lp >> p.cp_ishift;
        return (((run * p.cp_world) + p.cp_rank) << p.cp_ishift) + (lp & ((1 << p.cp_ishift) - 1));
      } else {
        return lp;
      }
    };

    // running softmax state of each query row
    float m_run[NC], l_run[NC];  // l_run: this lane's tokens only
    f32x4 acc[NC][NT];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      m_run[c] = -INFINITY;
      l_run[c] = 0.0f;
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[c][n] = (f32x4){0.f, 0.f, 0.f, 0.f};
    }

    // Scores, online softmax and P.V for one tile whose loads have landed.
    auto consume = [&](int tt, TileBuf& bf) {
      const bool active = bf.bid > 0;
      float sx[NC][4];  // scale_log2 * S^T[token 4*jg+i][row 16c+rho]
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int pp = 0; pp < NP; ++pp) {
          if constexpr (BF16) {
            s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, bf.k[pp]),
                                                        __builtin_bit_cast(bf16x8, qp[c][pp]), s,
                                                        0, 0, 0);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              s = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(bf.k[pp][e]),
                                                       __uint_as_float(qp[c][pp][e]), s, 0, 0, 0);
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) sx[c][i] = s[i] * p.scale_log2;
      }
      const bool full = active && (tt + kTile <= E) && (gpos(tt + kTile - 1) <= qpos_min) &&
                        (!GEN || tt >= all_lo);
      if (!full) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int pos = tt + 4 * jg + i;
          const bool kv_ok = active && pos < E;
          const int64_t gp = gpos(pos);
#pragma unroll
          for (int c = 0; c < NC; ++c)
            if (!(kv_ok && gp <= qpos[c] && (!GEN || pos >= qlo[c]))) sx[c][i] = -INFINITY;
          if (!kv_ok) {
#pragma unroll
            for (int w = 0; w < NVW; ++w) bf.v[i][w] = kNegZero;
          }
        }
      }

      // online softmax, per row. The row's exponent reference m_run moves only
      // when a tile's max passes it by more than 8 (log2 units), to that max:
      // the weights exp2(s - m_run) stay below 2^8, exact in the three-term
      // split and far from fp32 overflow in l and acc, and the accumulator
      // rescale (NT * 4 * NC multiplies) runs a few times per segment instead
      // of at most tiles. (m_run is a reference, not the running max; the
      // partial state and the merges use it as such.)
      float pr4[NC][4];
      bool moved = false;
      float alpha[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        float mx = fmaxf(fmaxf(sx[c][0], sx[c][1]), fmaxf(sx[c][2], sx[c][3]));
        mx = max_over_groups(mx);
        const float m_new = mx > m_run[c] + 8.0f ? mx : m_run[c];
        const float m_use = m_new == -INFINITY ? 0.0f : m_new;
        alpha[c] = __builtin_amdgcn_exp2f(m_run[c] - m_use);
#pragma unroll
        for (int i = 0; i < 4; ++i) pr4[c][i] = __builtin_amdgcn_exp2f(sx[c][i] - m_use);
        l_run[c] = l_run[c] * alpha[c] + ((pr4[c][0] + pr4[c][1]) + (pr4[c][2] + pr4[c][3]));
        m_run[c] = m_new;
        moved |= alpha[c] != 1.0f;
      }
      if (__any(moved)) {
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
          for (int n = 0; n < NT; ++n) acc[c][n] *= alpha[c];
      }

      // O^T += V^T P^T
      if constexpr (BF16) {
        // The whole tile at once: lane (jg, rho) gives A = V^T[dim column]
        // [tokens 4 jg .. 4 jg + 3] and B = P^T[those tokens][row 16 c + rho].
        // P is split into three bf16 terms, each the top 8 significant bits of
        // what the previous ones left (a truncation, so the remainder is
        // exact): hi + mid + lo == p bit for bit. Two v_mfma_f32_16x16x32_bf16
        // take them, each contraction running over the lane's four tokens
        // twice (A repeats the four values): B = (hi, mid), then (lo, 0); the
        // products accumulate in fp32. (Only this one MFMA kind touches the
        // accumulator: a 16x16x16 step chained to a 16x16x32 one on the same
        // accumulator got too few wait states from the compiler and read a
        // stale accumulator.)
        u32x4 pt_hm[NC], pt_l0[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          float rem[4] = {pr4[c][0], pr4[c][1], pr4[c][2], pr4[c][3]};
          u32x2 pt[3];
#pragma unroll
          for (int term = 0; term < 3; ++term) {
            pt[term] = (u32x2){bf16_pair_hi(rem[0], rem[1]), bf16_pair_hi(rem[2], rem[3])};
#pragma unroll
            for (int t = 0; t < 4; ++t)
              rem[t] -= __uint_as_float(__float_as_uint(rem[t]) & 0xffff0000u);
          }
          pt_hm[c] = (u32x4){pt[0][0], pt[0][1], pt[1][0], pt[1][1]};
          pt_l0[c] = (u32x4){pt[2][0], pt[2][1], 0u, 0u};
        }
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          // dimension column rho of n-tile n is dimension rho * NT + n: the
          // low or high half of dword n / 2 of each token's 16-byte slice
          const uint32_t sel = (n & 1) ? kPermHi : kPermLo;
          const uint32_t a01 = __builtin_amdgcn_perm(bf.v[1][n >> 1], bf.v[0][n >> 1], sel);
          const uint32_t a23 = __builtin_amdgcn_perm(bf.v[3][n >> 1], bf.v[2][n >> 1], sel);
          const bf16x8 a = __builtin_bit_cast(bf16x8, (u32x4){a01, a23, a01, a23});
#pragma unroll
          for (int c = 0; c < NC; ++c) {
            acc[c][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                a, __builtin_bit_cast(bf16x8, pt_hm[c]), acc[c][n], 0, 0, 0);
            acc[c][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                a, __builtin_bit_cast(bf16x8, pt_l0[c]), acc[c][n], 0, 0, 0);
          }
        }
      } else {
        // fp32 values on v_mfma_f32_16x16x4f32, four tokens per step: lane
        // (jg, rho) gives dimension column rho of token 4 jg + i
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
          for (int n = 0; n < NT; ++n)
#pragma unroll
            for (int c = 0; c < NC; ++c)
              acc[c][n] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(bf.v[i][n]),
                                                               pr4[c][i], acc[c][n], 0, 0, 0);
        }
      }
    };
    walk_tiles_of(p.block_table + (int64_t)r * p.table_stride, off, (t_lo + t0) * kTile,
                  (t_lo + t1) * kTile, consume, load_q);

    // acc[c][n][i] holds dimension (4*jg + i) * NT + n of query row row0 + 16c + rho.
    // Its float4 k = i * NT / 4 + n0 / 4 gathers n-tiles n0 .. n0 + 3 of
    // component i: dimensions d_base + i * NT + n0 .. + 3 of the row.
    auto own_vec = [&](int c, int k) -> f32x4 {
      const int i = k / (NT / 4), n0 = (k % (NT / 4)) * 4;
      return (f32x4){acc[c][n0][i], acc[c][n0 + 1][i], acc[c][n0 + 2][i], acc[c][n0 + 3][i]};
    };
    const int grp = (wave % NW) * RH + rh;  // the WS waves holding these rows
    auto mine = [&](int k) { return WS == 1 || k % WS == ws; };
    const int d_base = 4 * jg * NT;
    const bool whole = t0 == 0 && t1 == nr;
    if (t0 == 0 && hg == 0 && threadIdx.x == 0) {
      // Request r's partials sit at slots slice + r .. last slice + r.
      p.chunk_meta[2 * r] = slice + r;
      p.chunk_meta[2 * r + 1] = whole ? 1 : (pr + nr - 1) / Q - slice + 1;
    }
    float* pslot = p.partials + (((int64_t)slice + r) * Hkv + g) * nrows * PSTRIDE;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      // Tile split: the WS waves of a head pool their states of column tile c
      // in LDS. The merged state has the largest of their maxima; each wave's
      // state enters it scaled by 2^(its max - that max), summed in wave order
      // 0 .. WS-1. Every wave computes the merged (m, l) and the float4s k
      // with k mod WS == ws.
      float sc[WS];
      if constexpr (WS > 1) {
        // the previous column tile's pool is read (and, with traded halves,
        // the walk's last halves, which share its LDS)
        // (K through LDS: every wave's last loads into its ring, which the
        // pool overlays, have landed)
        if (KL && c == 0) __builtin_amdgcn_s_waitcnt(kVmcnt0);
        if (c > 0 || KL) __syncthreads();
        const int at = grp * WS + ws;
        s_pm[at * 64 + lane] = m_run[c];
        s_pl[at * 64 + lane] = l_run[c];
#pragma unroll
        for (int k = 0; k < NT; ++k) s_pool[(at * NT + k) * 64 + lane] = own_vec(c, k);
        __syncthreads();
        float ms[WS], mx = -INFINITY;
#pragma unroll
        for (int w = 0; w < WS; ++w) {
          ms[w] = s_pm[(grp * WS + w) * 64 + lane];
          mx = fmaxf(mx, ms[w]);
        }
        const float mu = mx == -INFINITY ? 0.0f : mx;  // no wave saw a key
        float l = 0.0f;
#pragma unroll
        for (int w = 0; w < WS; ++w) {
          sc[w] = __builtin_amdgcn_exp2f(ms[w] - mu);
          l = __builtin_fmaf(s_pl[(grp * WS + w) * 64 + lane], sc[w], l);
        }
        m_run[c] = mx;
        l_run[c] = l;
      }
      auto vec = [&](int k) -> f32x4 {
        if constexpr (WS == 1) {
          return own_vec(c, k);
        } else {
          f32x4 v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int w = 0; w < WS; ++w) {
            const f32x4 o = s_pool[((grp * WS + w) * NT + k) * 64 + lane];
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = __builtin_fmaf(o[e], sc[w], v[e]);
          }
          return v;
        }
      };
      const float l_tot = sum_over_groups(l_run[c]);  // whole-wave sum: every lane takes part
      const int row = row0 + 16 * c + rho;
      if (row < nrows && whole) {
        const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
        float* o =
            p.out + (((int64_t)r * Sq + jrow[c]) * Hq + (int64_t)g * G + hh[c]) * D + d_base;
#pragma unroll
        for (int k = 0; k < NT; ++k) {
          if (!mine(k)) continue;
          const int i = k / (NT / 4), n0 = (k % (NT / 4)) * 4;
          *(f32x4*)(o + i * NT + n0) = vec(k) * inv;
        }
        if (p.lse_out && jg == 0 && ws == 0)
          p.lse_out[((int64_t)r * Sq + jrow[c]) * Hq + (int64_t)g * G + hh[c]] =
              row_lse(m_run[c], l_tot);
      } else if (row < nrows) {
        // split: publish this segment's partial state, in store order: float4
        // k of lane (jg, row) sits at float4 index (k * 4 + jg) * nrows + row of
        // the slot, so each store writes contiguous runs of 16 rows (a row-major
        // layout would put each lane's 16 bytes in a different cache line);
        // (m, l) of the rows follow all the float4s.
#pragma unroll
        for (int k = 0; k < NT; ++k) {
          if (!mine(k)) continue;
          *(f32x4*)(pslot + ((k * 4 + jg) * nrows + row) * 4) = vec(k);
        }
        if (jg == 0 && ws == 0) *(f32x2*)(pslot + nrows * D + 2 * row) = (f32x2){m_run[c], l_tot};
      }
    }
  };

  // ---- this slice's context tiles, request by request ---------------------
  {
    int r = uniform(s_first[0]);
    int pos = a;
    while (pos < b) {
      const int pr = uniform(s_pref[r]);
      const int pn = uniform(s_pref[r + 1]);
      if (pn > pos) {
        const int e = min(b, pn);
        const int t_base = pr + X;  // unit of r's tile 0
        const int t0 = max(pos, t_base) - t_base;
        const int t1 = e - t_base;
        if (t1 > t0) segment(r, t0, t1, pn - t_base, t_base);
        pos = e;
      }
      ++r;
    }
  }

  // ---- requests with no visible context produce zeros --------------------
  for (int r = blockIdx.x; r < B; r += gridDim.x) {
    if (s_pref[r + 1] == s_pref[r]) {
      const int row_floats = Sq * Hq * D;
      float* o = p.out + (int64_t)r * row_floats;
      for (int i = threadIdx.x; i < row_floats; i += NTHR) o[i] = 0.0f;
      if (p.lse_out)
        for (int i = threadIdx.x; i < Sq * Hq; i += NTHR) p.lse_out[(int64_t)r * Sq * Hq + i] = -INFINITY;
      if (threadIdx.x == 0) p.chunk_meta[2 * r + 1] = 0;
    }
  }

  // ---- fixed-shape walk: read this slice's padding tiles, use none -------
  if constexpr (TW) {
    auto drain = [&](int, TileBuf& bf) {
#pragma unroll
      for (int pp = 0; pp < NP; ++pp) sink ^= bf.k[pp][0] ^ bf.k[pp][1] ^ bf.k[pp][2] ^ bf.k[pp][3];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int w = 0; w < NVW; ++w) sink ^= bf.v[i][w];
    };
    int r = uniform(s_first[1]);
    int tp = uniform(s_first[2]);  // context tiles of the requests before r
    int pos = pa;
    while (pos < pbnd) {
      const int wu = uniform(s_pref[r + 1]) - uniform(s_pref[r]);
      const int n = wu > 0 ? wu - X : 0;
      const int pr = r * walk_tiles - tp;
      const int pn = pr + (walk_tiles - n);
      if (pn > pos) {
        const int e = min(pbnd, pn);
        walk_tiles_of(p.block_table + (int64_t)r * p.table_stride, 0, (n + pos - pr) * kTile,
                      (n + e - pr) * kTile, drain, [] {});
        pos = e;
      }
      tp += n;
      ++r;
    }
    if (p.flags & kFlagSink) p.out[0] = __uint_as_float(sink);
  }
  // no load into this workgroup's LDS outlives it
  if constexpr (KL) __builtin_amdgcn_s_waitcnt(kVmcnt0);
}

// Workgroups of a kernel the device holds at once (compute units times
// workgroups per unit at that size and LDS), queried once per device and
// kernel; `cache` is the kernel's per-device slot.
constexpr int kMaxDevices = 64;

inline hipError_t resident_of(const void* kernel, int threads, size_t lds,
                       std::atomic<int> (&cache)[kMaxDevices], int* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const bool cached = dev >= 0 && dev < kMaxDevices;
  if (cached && (*out = cache[dev].load(std::memory_order_relaxed)) > 0) return hipSuccess;
  int cus = 0, per_cu = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, lds);
  if (e != hipSuccess) return e;
  *out = (cus > 0 ? cus : 1) * (per_cu > 0 ? per_cu : 1);
  if (cached) cache[dev].store(*out, std::memory_order_relaxed);
  return hipSuccess;
}

// Pass-1 workgroups at the largest LDS the kernel asks for. The context
// walk's figure serves every mode, so all modes cut the batch the same way.
template <bool BF16, int D, int NW, int NC, int RH, int WS>
hipError_t resident_workgroups(int* out) {
  static std::atomic<int> cache[kMaxDevices];
  return resident_of(
      reinterpret_cast<const void*>(&paged_decode_kernel<BF16, D, NW, kContextWalk, NC, RH, WS>),
      NW * RH * WS * 64, decode_lds_bytes(kDecodeMaxSeqs), cache, out);
}

// Compute units of the current device, queried once per device.
inline hipError_t device_cus(int* out) {
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const bool cached = dev >= 0 && dev < kMaxDevices;
  if (cached && (*out = cache[dev].load(std::memory_order_relaxed)) > 0) return hipSuccess;
  e = hipDeviceGetAttribute(out, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  if (*out < 1) *out = 1;
  if (cached) cache[dev].store(*out, std::memory_order_relaxed);
  return hipSuccess;
}

// The slices the batch's tiles are cut into on the current device: one per
// resident workgroup slot (per head group), at most eight waves per compute
// unit (more waves add partials to merge but no bytes in flight that the
// stream needs) and one workgroup per compute unit at four KV heads per
// workgroup (4 waves: measured 4-6% faster than two such workgroups per
// unit, while two-head workgroups are fastest at four per unit), never more
// than the workspace holds partials for.
template <bool BF16, int D, int NW, int NC, int RH, int WS>
hipError_t slices_typed(const DecodeParams& p, int* slices) {
  constexpr int waves = NW * RH * WS;
  const int HG = p.num_kv_heads / NW;
  int resident = 0, cus = 0;
  hipError_t e = resident_workgroups<BF16, D, NW, NC, RH, WS>(&resident);
  if (e != hipSuccess) return e;
  e = device_cus(&cus);
  if (e != hipSuccess) return e;
  const int cap = cus * (NW == 4 && RH == 1 && WS == 1 ? 1 : (waves >= 8 ? 1 : 8 / waves));
  const int wgs = resident < cap ? resident : cap;
  int s = wgs / HG > 1 ? wgs / HG : 1;
  if (s > p.max_slices) s = p.max_slices;
  *slices = s;
  return hipSuccess;
}

// Pass 1 over p.slices slices (the caller's cut): the step's writes first
// when they do not qualify for the append mode, then the kernel of the
// walk mode.
template <bool BF16, int D, int NW, int NC, int RH, int WS>
hipError_t pass1_typed(const DecodeParams& p, int bs_shift, hipStream_t stream) {
  constexpr int NTHR = NW * RH * WS * 64;
  const int HG = p.num_kv_heads / NW;
  const dim3 grid((unsigned)p.slices * (unsigned)HG);
  const size_t lds = decode_lds_bytes(p.num_seqs);
  hipError_t e;
  if (p.app_max_tokens > 0) {
    // The step's rows are written by pass 1 when all its tokens fit one
    // workgroup's threads and the walk is the context walk; otherwise by
    // the fused slot-map + write kernel first.
    if (!(p.flags & kFlagWalkTable) && p.window == 0 && !p.kv_pos_offset && p.cp_world == 1 &&
        p.app_max_tokens <= NTHR) {
      paged_decode_kernel<BF16, D, NW, kAppend, NC, RH, WS>
          <<<grid, dim3(NTHR), lds, stream>>>(p, bs_shift);
      return hipGetLastError();
    }
    e = launch_slot_write(p.app_req, p.app_pos, p.app_tokens, p.app_max_tokens, p.block_table,
                          p.num_seqs, p.table_stride, p.block_size, p.app_slots, p.app_k,
                          p.app_v, p.app_k_cache, p.app_v_cache, p.total_blocks * p.block_size,
                          p.num_kv_heads * p.head_dim * (p.is_bf16 ? 2 : 4), stream);
    if (e != hipSuccess) return e;
  }
  if (p.flags & kFlagWalkTable)
    paged_decode_kernel<BF16, D, NW, kTableWalk, NC, RH, WS>
        <<<grid, dim3(NTHR), lds, stream>>>(p, bs_shift);
  else if (p.window > 0 || p.kv_pos_offset || p.cp_world > 1)
    paged_decode_kernel<BF16, D, NW, kGeneral, NC, RH, WS>
        <<<grid, dim3(NTHR), lds, stream>>>(p, bs_shift);
  else
    paged_decode_kernel<BF16, D, NW, kContextWalk, NC, RH, WS>
        <<<grid, dim3(NTHR), lds, stream>>>(p, bs_shift);
  return hipGetLastError();
}

// Up to 16 rows per KV head (one column tile) of a bf16 cache: workgroups of
// eight waves, two KV heads with four waves each splitting the tiles (one
// head with eight when Hkv is odd). Measured against one wave per head and
// eight heads per workgroup: the 256-request batch 656 vs 682 us, the 64
// ragged requests 352 vs 371 us, bucketing 63.9 vs 66.1 us, the 4-rank
// context-parallel share 197 vs 205 us, the 12-request batch 31.9 vs 30.9 us;
// four heads of two waves each were no faster than eight of one.
// Otherwise: one wave per head for the rows of up to 32 (RH = 1) and the
// largest of 8, 4, 2, 1 heads dividing Hkv; two per head for up to 64 rows
// (RH = 2, at most four heads). (At two column tiles, and with fp32 values,
// the pooled merge's registers would spill.)
template <bool BF16, int NC, int RH>
constexpr bool tile_split = BF16;

template <bool BF16, int D, int NC, int RH>
hipError_t pass1_heads(const DecodeParams& p, int bs_shift, hipStream_t stream) {
  const int h = p.num_kv_heads;
  if constexpr (tile_split<BF16, NC, RH>) {
    if (h % 2 == 0) return pass1_typed<BF16, D, 2, NC, RH, 4 / RH>(p, bs_shift, stream);
    return pass1_typed<BF16, D, 1, NC, RH, 8 / RH>(p, bs_shift, stream);
  } else {
    if constexpr (RH == 1) {
      if (h % 8 == 0) return pass1_typed<BF16, D, 8, NC, RH, 1>(p, bs_shift, stream);
    }
    if (h % 4 == 0) return pass1_typed<BF16, D, 4, NC, RH, 1>(p, bs_shift, stream);
    if (h % 2 == 0) return pass1_typed<BF16, D, 2, NC, RH, 1>(p, bs_shift, stream);
    return pass1_typed<BF16, D, 1, NC, RH, 1>(p, bs_shift, stream);
  }
}

template <bool BF16, int D, int NC, int RH>
hipError_t slices_heads(const DecodeParams& p, int* slices) {
  const int h = p.num_kv_heads;
  if constexpr (tile_split<BF16, NC, RH>) {
    if (h % 2 == 0) return slices_typed<BF16, D, 2, NC, RH, 4 / RH>(p, slices);
    return slices_typed<BF16, D, 1, NC, RH, 8 / RH>(p, slices);
  } else {
    if constexpr (RH == 1) {
      if (h % 8 == 0) return slices_typed<BF16, D, 8, NC, RH, 1>(p, slices);
    }
    if (h % 4 == 0) return slices_typed<BF16, D, 4, NC, RH, 1>(p, slices);
    if (h % 2 == 0) return slices_typed<BF16, D, 2, NC, RH, 1>(p, slices);
    return slices_typed<BF16, D, 1, NC, RH, 1>(p, slices);
  }
}

// NC column tiles per wave, RH waves per KV head (16 NC RH query rows).
template <int NC, int RH>
hipError_t pass1_for(const DecodeParams& p, hipStream_t stream) {
  const int bs_shift = __builtin_ctz((unsigned)p.block_size);
  if (p.is_bf16) {
    if (p.head_dim == 128) return pass1_heads<true, 128, NC, RH>(p, bs_shift, stream);
    return pass1_heads<true, 64, NC, RH>(p, bs_shift, stream);
  }
  if (p.head_dim == 128) return pass1_heads<false, 128, NC, RH>(p, bs_shift, stream);
  return pass1_heads<false, 64, NC, RH>(p, bs_shift, stream);
}

template <int NC, int RH>
hipError_t slices_for(const DecodeParams& p, int* slices) {
  if (p.is_bf16) {
    if (p.head_dim == 128) return slices_heads<true, 128, NC, RH>(p, slices);
    return slices_heads<true, 64, NC, RH>(p, slices);
  }
  if (p.head_dim == 128) return slices_heads<false, 128, NC, RH>(p, slices);
  return slices_heads<false, 64, NC, RH>(p, slices);
}

}  // namespace

// Pass 1 (and the slices it cuts the batch into) at up to 16, 32 and 64
// query rows per KV head (one wave of one column tile, one wave of two, two
// waves of two), one translation unit each (paged_decode.hip,
// paged_decode_nc2.hip, paged_decode_nc4.hip).
hipError_t decode_pass1_nc1(const DecodeParams& p, hipStream_t stream);
hipError_t decode_pass1_nc2(const DecodeParams& p, hipStream_t stream);
hipError_t decode_pass1_nc4(const DecodeParams& p, hipStream_t stream);
hipError_t decode_slices_nc1(const DecodeParams& p, int* slices);
hipError_t decode_slices_nc2(const DecodeParams& p, int* slices);
hipError_t decode_slices_nc4(const DecodeParams& p, int* slices);

}  // namespace kvs
