// Ragged causal prefill on bf16 matrix cores (gfx950), with the MLA split
// head and an optional 64x64 block-sparse mask.
//
// What is computed (Modular flare_mla_prefill; FlashMLA tensor-shape
// reference, section 3): sequences are packed back to back (cu_seqlens);
// query i of a sequence sees key j iff j <= i and, with a block mask,
// mask[b, i/64, j/64] != 0.  The score of query head h and key j is
//   scale * (q[i,h,:Dn] . k[j,g,:] + q[i,h,Dn:] . k_rope[j,0,:]),  g = h/(Hq/Hk),
// i.e. the rope part of the key is one 64-wide row shared by every head.  The
// output has the value width (128).
//
// Work split: one workgroup of four waves per (sequence, query head, 128-row
// query tile), or, with a block mask and Hq / Hk even, per (sequence, pair of
// heads of one KV group, 64-row query tile); each wave owns 32 query rows of
// one head.  Key tiles of 64 rows (K, the
// shared rope K and V) are staged into XOR-swizzled LDS through registers,
// double-buffered so the next tile's loads are in flight during the current
// tile's math.  Scores are formed transposed, S^T = K Q^T, on
// v_mfma_f32_32x32x16_bf16 (K rows from LDS as the A operand, the wave's Q
// held in registers as the B operand), so each lane holds one query's
// scores and the row softmax needs a single cross-lane exchange.  O^T =
// V^T P^T runs on the same MFMA with V^T delivered by the LDS transpose
// read.  Tiles that the causal order or the block mask hide from both query
// blocks of the workgroup are never loaded; a wave skips the math of tiles
// hidden from its own rows.  Workgroups are dispatched deepest query tile
// first, and the heads of one KV group are placed on one XCD so that their
// shared K/V stay in that XCD's L2.
#include "dev.hpp"
#include "status.hpp"

#include <algorithm>
#include <cmath>
#include <type_traits>

namespace gqap {

struct PrefillArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* kr;
  const int32_t* cu;
  const uint8_t* mask;
  uint16_t* out;
  float* lse;
  int64_t q_st, q_sh, k_st, k_sh, v_st, v_sh, kr_st, o_st, o_sh;
  int32_t B, Hq, Hk, ratio, q_tiles, mask_nb, max_len;
  int32_t hpw;       // heads per workgroup: 1 (128 query rows of one head) or
                     // 2 (64 rows of two heads of one KV group)
  float scale_log2;  // scale * log2(e)
  // Chunked prefill against the paged cache: k and v are the pools, the
  // query rows of sequence b are the last of its kvlens[b] keys.
  const int32_t* kvlens;
  const int32_t* bt;
  int64_t bt_st;      // block_table row stride (int32 elements)
  int64_t kv_sb;      // elements between pool blocks
  int64_t kv_sh;      // elements between heads of a block
  int64_t kr_sb;      // elements between rope-cache blocks
  int32_t max_kv;     // capacity: keys per sequence
  // fp8 prefill: q and k hold e4m3fn codes of the nope parts (strides in
  // bytes), the rope part of the query is the bf16 tensor qr, and the nope
  // term of a score is multiplied by qk = q_scale * k_scale.
  const uint16_t* qr;
  int64_t qr_st, qr_sh;
  float qk;
  // fp8 prefill with blockwise scales: one float per row of a head,
  // q_scale [T, Hq] and k_scale [T, Hk], both contiguous.
  const float* qsc;
  const float* ksc;
  // Split over the key axis: with nsplit > 1 each query tile is processed by
  // nsplit workgroups, one contiguous range of its key tiles each, and they
  // write normalised fp32 partials (ws_o [nsplit][T][Hq][128], ws_lse
  // [nsplit][T][Hq], natural log) that prefill_merge combines.
  int32_t nsplit;
  int32_t T;
  // Paged grids of more than one round of workgroups: items ranked by the
  // keys their last row sees (see the kernel), else by query tile.
  int32_t rank_keys;
  float* ws_o;
  float* ws_lse;
  // fp8 KV pages: the value of a V code is e4m3fn(code) * v_scale; k_scale is
  // folded into scale_log2 without a rope part, else held in qk and applied
  // to the nope sum only (the rope cache is bf16 and unscaled).
  float v_scale;
};

namespace dev {

typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;

__device__ __forceinline__ f32x16_t mfma32x32x16(bf16x8 a, bf16x8 b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// D += A B on fp8 e4m3fn operands (format code 0 for both), 64-deep: each lane
// brings 32 codes.  Zero scale operands select the unscaled instruction
// v_mfma_f32_32x32x64_f8f6f4.  The products of two e4m3fn values are exact in
// fp32.  The output layout is that of the bf16 32x32 step, and a k order that
// is the same for both operands gives the plain dot product.
__device__ __forceinline__ f32x16_t mfma32x32x64_fp8(i32x8 a, i32x8 b, f32x16_t c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Eight OCP e4m3fn bytes (little-endian in w) -> eight bf16 values, two per
// instruction with the gfx950 scaled conversion at scale 1 (exact: every
// e4m3fn value is a bf16 value).
__device__ __forceinline__ i32x4 fp8x8_to_bf16x8_pk(i32x2 w) {
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
  i32x4 r;
  r[0] = __builtin_bit_cast(int, (bf16x2)__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)w[0], 1.f, false));
  r[1] = __builtin_bit_cast(int, (bf16x2)__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)w[0], 1.f, true));
  r[2] = __builtin_bit_cast(int, (bf16x2)__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)w[1], 1.f, false));
  r[3] = __builtin_bit_cast(int, (bf16x2)__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)w[1], 1.f, true));
  return r;
}

// 16-byte chunk c of row `row` of a tile with RC chunks per row, XOR-swizzled
// so that 16 consecutive rows read at one logical chunk hit distinct banks.
template <int RC>
__device__ __forceinline__ int kswz(int row, int c) {
  if constexpr (RC >= 16) {
    return row * RC * 16 + ((c ^ (row & 15)) << 4);
  } else {  // RC == 8: two rows per 256-byte bank window
    return row * RC * 16 + ((c ^ ((row >> 1) & 7)) << 4);
  }
}

// V tile (64 rows x 256 bytes): 32-byte pieces XOR-permuted by a function
// of the row.  A transpose read has four 16-lane groups; groups 0 and 1 read
// rows 8k..8k+3 at pieces P and P^1, groups 2 and 3 rows 8k+4..8k+7.  The
// mask 2*(row & 3) + ((row >> 2) & 1) sends the first two groups to the even
// and the odd pieces respectively, so each half-wave covers all 64 banks.
__device__ __forceinline__ int vmask(int row) { return 2 * (row & 3) + ((row >> 2) & 1); }
__device__ __forceinline__ int vswz256(int row, int c) {
  return row * 256 + (((c >> 5) ^ vmask(row)) << 5) + (c & 31);
}

}  // namespace dev

using namespace dev;

// F8 = 1 or 2: the nope parts of Q and K are fp8 e4m3fn codes (K tiles of 64
// rows x 128 bytes, staged like the rope tile) and their products run on the
// fp8 matrix cores; the rope parts and V stay bf16.  F8 = 1 has one scale per
// tensor, F8 = 2 one per row of a head (the key scales of a tile are staged in
// LDS next to it).
// F8 = 3 (paged only): the K and V pages hold fp8 e4m3fn codes with
// per-tensor scales.  Each page is loaded into registers, widened exactly to
// bf16 (every e4m3fn value is a bf16 value) and written to the LDS layouts of
// a bf16 tile, so the math is that of the bf16 path; k_scale is part of the
// softmax constant and v_scale multiplies the normalised output.
// F8 = 4 (ragged MLA only): the shared rope keys are fp8 e4m3fn codes with
// one scale per row (token).  The rope tile is staged as 64-byte code rows
// with its 64 scales; a rope operand is widened exactly to bf16 when it is
// read, each half tile runs its rope steps first, multiplies that sum by the
// keys' scales, then accumulates the bf16 per-head steps.
// Sum over a wave of per-lane counts in [0, 2^nb): one ballot per bit, so no
// data moves between lanes (each step is a compare and a bit count).
__device__ __forceinline__ int wave_sum_small(int v, int nb) {
  int t = 0;
  for (int k = 0; k < nb; ++k) t += __builtin_popcountll(__ballot((v >> k) & 1)) << k;
  return t;
}

template <int DR, bool PAGED, int F8>
__global__ __launch_bounds__(256, 2) void prefill_fwd(PrefillArgs a) {
  constexpr bool QK8 = F8 == 1 || F8 == 2;    // fp8 nope Q.K on the fp8 matrix cores
  constexpr bool KV8 = F8 == 3;               // fp8 KV pages, widened to bf16 in LDS
  constexpr bool RK8 = F8 == 4;               // fp8 rope keys with per-row scales
  constexpr bool KSC = F8 == 2 || RK8;        // per-key scales staged in LDS with each tile
  static_assert(!(QK8 && PAGED), "the fp8 Q.K path reads token-major K");
  static_assert(!KV8 || PAGED, "the fp8 KV path reads pages");
  static_assert(!RK8 || (DR == 64 && !PAGED), "fp8 rope keys: ragged MLA prefill");
  constexpr int DN = 128;                     // per-head key width
  constexpr int DV = 128;                     // value / output width
  constexpr int KSN = DN / 16;                // k-steps over the nope part (bf16)
  constexpr int KSR = DR / 16;                // k-steps over the rope part
  constexpr int KE = QK8 ? 1 : 2;             // bytes per K element in LDS
  constexpr int KGE = QK8 || KV8 ? 1 : 2;     // bytes per K element in memory
  constexpr int VGE = KV8 ? 1 : 2;            // bytes per V element in memory
  constexpr int KB = 64 * DN * KE;            // K tile bytes
  constexpr int RB = DR ? 64 * DR * (RK8 ? 1 : 2) : 0;  // rope tile bytes
  constexpr int VB = 64 * DV * 2;             // V tile bytes
  // Loads per lane and tile: 16-byte loads-to-LDS (1 KB per wave each), or
  // with KV8 16-byte register loads of codes (two per lane for K, two for V).
  constexpr int KLD = KV8 ? 2 : KB / 1024 / 4;  // K
  constexpr int RLD = RB / 1024 / 4;            // rope
  constexpr int VLD = KV8 ? 2 : VB / 1024 / 4;  // V
  // LDS: one array per tile buffer, so the compiler can tell the buffer being
  // filled by the direct-to-LDS loads from the one being read.
  __shared__ __attribute__((aligned(1024))) unsigned char kbuf0[KB], kbuf1[KB];
  __shared__ __attribute__((aligned(1024))) unsigned char rbuf0[RB ? RB : 16], rbuf1[RB ? RB : 16];
  __shared__ __attribute__((aligned(1024))) unsigned char vbuf0[VB], vbuf1[VB];
  // Blockwise key scales of a tile: one 64-float copy per wave.
  __shared__ __attribute__((aligned(1024))) float sbuf0[KSC ? 256 : 4], sbuf1[KSC ? 256 : 4];

  // Work item.  The grid is one-dimensional, Hq / hpw workgroups (times the
  // key-axis splits) per (query tile, sequence) item.  Items are ranked
  // deepest query tile first, then by sequence; a paged grid of more than
  // one round of workgroups (up to 64 sequences) ranks them instead by the
  // keys their last row sees, most first, since there the cached prefixes,
  // not the query tile, set an item's length and the longest must start
  // first.  Only items that exist (query tile inside its sequence) are
  // ranked, so all real work precedes the empty tail of the grid and is
  // spread evenly over the dispatcher's shader engines.  Within an item the heads of one KV group share an XCD
  // (workgroup i runs on XCD i % 8).
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  // With hpw = 2 the workgroup's unit is a pair of heads of one KV group,
  // waves 0-1 taking 64 query rows of the first head and waves 2-3 the same
  // rows of the second, so that all four waves see the same key tiles.
  const int NH = a.Hq / a.hpw;                     // workgroups per item and split
  const int QT = 128 / a.hpw;                      // query rows per workgroup and head
  const int x = blockIdx.x % NH;
  const int sp = (blockIdx.x / NH) % a.nsplit;     // key-axis split
  const int item = blockIdx.x / NH / a.nsplit;
  const int hpx = NH >> 3;
  const int hx = (NH & 7) ? x : (x & 7) * hpx + (x >> 3);  // head, or head pair
  const int h = a.hpw == 2 ? 2 * hx + (wv >> 1) : hx;      // this wave's head
  const int wslot = a.hpw == 2 ? (wv & 1) : wv;            // this wave's 32-row slot
  // Query tiles of a sequence of Lq query rows: those of its first max_len
  // rows, and all of the plan's tiles when it is longer (the last of them
  // then also clears the rows past the capacity).
  auto item_tiles = [&](int Lq) {
    return Lq <= 0 ? 0 : Lq > a.max_len ? a.q_tiles : (Lq + QT - 1) / QT;
  };
  int b, qt;
  if (PAGED && a.rank_keys && a.B <= 64) {
    // Lane l holds sequence l: its query rows, query tiles and key offset
    // (cached keys before the chunk).  Item (b, qt) costs about as many key
    // tiles as its last row sees keys, off + min(Lq, (qt + 1) QT): a value
    // that grows strictly with qt, so a sequence has at most one item per
    // value.  Items are ranked by that value, largest first (ties by
    // sequence), so the longest items start first and the grid's end holds
    // the shortest ones.
    int nq = 0, lq = 0, koff = 0;
    if (lane < a.B) {
      lq = a.cu[lane + 1] - a.cu[lane];
      nq = item_tiles(lq);
      if constexpr (PAGED) koff = max(0, a.kvlens[lane] - lq);
    }
    // Sums of per-lane counts in [0, 2^nb) by one ballot per bit (no
    // cross-lane data movement: each step is a compare and a bit count).
    const int nb = 32 - __builtin_clz((unsigned)a.q_tiles | 1u);  // per-lane counts < 2^nb
    auto wave_sum = [&](int v) { return wave_sum_small(v, nb); };
    auto wave_max = [](int v) {
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o));
      return v;
    };
    const int qsh = a.hpw == 2 ? 6 : 7;  // log2 QT
    // items of this lane's sequence whose key count exceeds v
    auto deeper = [&](int v) {
      const int y = v - koff;  // need min(lq, (qt + 1) QT) > y
      if (nq == 0 || lq <= y) return 0;
      return y < 0 ? nq : max(0, nq - (y >> qsh));
    };
    if (item >= wave_sum(nq)) return;  // past the last real item
    // The key count v of rank `item`: the smallest v with at most `item`
    // items above it.
    int lo = -1, hi = wave_max(lane < a.B ? koff + lq : 0);
    while (hi - lo > 1) {
      const int mid = lo + ((hi - lo) >> 1);
      if (wave_sum(deeper(mid)) <= item) hi = mid; else lo = mid;
    }
    const int above = wave_sum(deeper(hi));
    const int at_v = deeper(hi - 1);  // this lane's items with count >= hi
    uint64_t m = __ballot(at_v > deeper(hi));
    for (int k = item - above; k > 0; --k) m &= m - 1;  // drop the lower set bits
    b = __builtin_amdgcn_readfirstlane(__builtin_ctzll(m));
    qt = __builtin_amdgcn_readfirstlane(__shfl(nq - at_v, b));  // uniform: keeps what follows scalar
  } else if (a.B <= 64) {
    // Deepest query tile first, then by sequence: one ballot per tile
    // index.  Without cached keys this is the key-count order up to ties,
    // and a single round of workgroups starts together in any order.
    int nq = 0;  // query tiles of sequence `lane`
    if (lane < a.B) nq = item_tiles(a.cu[lane + 1] - a.cu[lane]);
    b = -1;
    qt = -1;
    if (a.q_tiles > 32 && a.B * ((a.q_tiles + 63) >> 6) < a.q_tiles) {
      // Many tile indices (the walk below would take one dependent ballot
      // per index, which a workgroup starting beside a busy one issues
      // slowly: 8-10 us for the last items of a 128-index block-sparse grid).
      // C(t) = sum_b max(0, nq_b - t) items have a tile index >= t; it falls
      // with t, so the item's tile index is one less than the number of t
      // with C(t) > item.  Lane j evaluates t = j (+ 64, ...) from the
      // sequences' tile counts read one by one as scalars: about 4 B
      // instructions per 64 tile indices.
      int above = 0;
      for (int base = 0; base < a.q_tiles; base += 64) {
        const int j = base + lane;
        int c = 0;
        for (int s = 0; s < a.B; ++s) c += max(0, __builtin_amdgcn_readlane(nq, s) - j);
        above += __builtin_popcountll(__ballot(j < a.q_tiles && c > item));
      }
      if (above == 0) return;  // past the last real item
      qt = above - 1;
      const int before = wave_sum_small(max(0, nq - above), 32 - __builtin_clz((unsigned)a.q_tiles | 1u));
      uint64_t m = __ballot(nq > qt);
      for (int k = item - before; k > 0; --k) m &= m - 1;  // drop the lower set bits
      b = __builtin_ctzll(m);
    } else {
      int before = 0;
      for (int t = a.q_tiles - 1; t >= 0; --t) {
        uint64_t m = __ballot(nq > t);
        const int cnt = __builtin_popcountll(m);
        if (item < before + cnt) {
          for (int k = item - before; k > 0; --k) m &= m - 1;  // drop the lower set bits
          b = __builtin_ctzll(m);
          qt = t;
          break;
        }
        before += cnt;
      }
      if (qt < 0) return;  // past the last real item
    }
  } else {
    b = item % a.B;
    qt = a.q_tiles - 1 - item / a.B;
  }
  const int c0 = a.cu[b];
  const int Lq = a.cu[b + 1] - c0;             // query rows of the sequence
  const int nqb = item_tiles(Lq);
  if (qt >= nqb) return;
  int L = min(Lq, a.max_len);                  // rows computed: those within the plan's capacity
  // Keys: the sequence itself, or with PAGED its Lk cached keys, the query
  // rows being the last Lq of them (offset off = Lk - Lq), so query i sees
  // key j iff j <= off + i.  A chunk whose keys exceed the capacity, or that
  // is longer than its keys, has no row computed.
  int Lk = L, off = 0;
  if constexpr (PAGED) {
    Lk = a.kvlens[b];
    if (Lk > a.max_kv || Lk < Lq) L = Lk = 0;
    off = Lk - Lq;
  }
  // Rows that are not computed get out = 0 and lse = -inf, written once, by
  // split 0 of the sequence's last query tile, for the workgroup's heads.
  if (Lq > L && sp == 0 && qt == nqb - 1) {
    const int64_t pieces = (int64_t)(Lq - L) * a.hpw * 16;  // 16-byte pieces of 256-byte rows
    for (int64_t e = tid; e < pieces; e += 256) {
      const int64_t rh = e >> 4;
      const int row = L + (int)(rh / a.hpw);
      const int hz = a.hpw * hx + (int)(rh % a.hpw);
      store16(a.out + (int64_t)(c0 + row) * a.o_st + (int64_t)hz * a.o_sh + 8 * (e & 15), i32x4{0, 0, 0, 0});
      if (a.lse && (e & 15) == 0) a.lse[(int64_t)(c0 + row) * a.Hq + hz] = -INFINITY;
    }
  }
  const int q0 = qt * QT;
  if (q0 >= L) return;
  const int g = a.hpw * hx / a.ratio;        // KV head: the same for both heads of a pair

  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int r0 = q0 + 32 * wslot;            // first query row of this wave (local)
  const int qrow = r0 + l32;                 // this lane's query row
  const bool wave_rows = r0 < L;
  const int rlast = min(L, r0 + 32) - 1;     // last valid row of the wave
  const int klast = off + rlast;             // last key visible to the wave
  // Factor of the fp8 nope sum that belongs to this lane's query row: its
  // blockwise scale (the key's comes per score), or q_scale * k_scale.
  float qsl = 0.f;
  if constexpr (F8 == 2) qsl = qrow < L ? a.qsc[(int64_t)(c0 + qrow) * a.Hq + h] : 0.f;
  if constexpr (F8 == 1) qsl = a.qk;

  // The wave's queries as the B operand: lane (query l32, half hh) holds
  // d = 16 s + 8 hh .. +7 for k-step s (s < KSN: nope part, then rope).
  // With fp8 Q.K (F8 = 1, 2) the nope part is instead two 32-byte operands
  // of the fp8 step, lane (l32, hh) holding codes 64 s + 32 hh .. +31 for
  // step s, and qop holds only the bf16 rope part, read from its own tensor.
  constexpr int NQ = QK8 ? KSR : KSN + KSR;
  bf16x8 qop[NQ > 0 ? NQ : 1];
  i32x8 q8[2];
  {
    const bool ok = qrow < L;
    const int64_t tok = c0 + (ok ? qrow : 0);
    if constexpr (QK8) {
      const unsigned char* qp = (const unsigned char*)a.q + tok * a.q_st + (int64_t)h * a.q_sh + 32 * hh;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const i32x4 lo = load16(qp + 64 * s), hi = load16(qp + 64 * s + 16);
        q8[s] = ok ? __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7) : i32x8{};
      }
      if constexpr (DR > 0) {
        const uint16_t* rp = a.qr + tok * a.qr_st + (int64_t)h * a.qr_sh + 8 * hh;
#pragma unroll
        for (int s = 0; s < KSR; ++s) {
          const i32x4 v = load16(rp + 16 * s);
          qop[s] = __builtin_bit_cast(bf16x8, ok ? v : i32x4{0, 0, 0, 0});
        }
      }
    } else {
      const uint16_t* qp = a.q + tok * a.q_st + (int64_t)h * a.q_sh + 8 * hh;
#pragma unroll
      for (int s = 0; s < KSN + KSR; ++s) {
        const i32x4 v = load16(qp + 16 * s);
        qop[s] = __builtin_bit_cast(bf16x8, ok ? v : i32x4{0, 0, 0, 0});
      }
    }
  }

  // Key tiles this workgroup must visit: keys < min(Lk, off + q0 + QT).
  const int nkt = max(0, min(Lk, off + q0 + QT) + 63) >> 6;
  // This workgroup's share of them: tiles [kt_begin, kt_end).
  const int kt_begin = (int)((int64_t)nkt * sp / a.nsplit);
  const int kt_end = (int)((int64_t)nkt * (sp + 1) / a.nsplit);
  const int qb0 = q0 >> 6;                   // the workgroup's query blocks (one with hpw = 2)
  const int qb1 = min((q0 + QT - 1) >> 6, (L - 1) >> 6);
  const int wqb = r0 >> 6;                   // this wave's query block
  // Tile schedule as bit words: bit i of word w is key tile 64 w + i.  `need`
  // = loaded by the workgroup (either query block sees it), `see` = this
  // wave's own query block sees it (mask part only).  Built with one load
  // per lane and a ballot once per 64 tiles, so the tile loop itself never
  // waits on memory for the mask.
  uint64_t need_word = 0, see_word = 0;
  int word_idx = -1;
  auto load_words = [&](int wi) {
    const int kt = wi * 64 + lane;
    bool need = kt < nkt, see = kt < nkt;
    if (a.mask && kt < nkt) {
      const uint8_t* mb = a.mask + (int64_t)b * a.mask_nb * a.mask_nb;
      const bool v0 = kt <= qb0 && mb[(int64_t)qb0 * a.mask_nb + kt];
      const bool v1 = kt <= qb1 && mb[(int64_t)qb1 * a.mask_nb + kt];
      need = v0 || v1;
      // (a wave whose rows all lie past the sequence end has no mask row)
      see = wave_rows && kt <= wqb && mb[(int64_t)wqb * a.mask_nb + kt];
    }
    need_word = __ballot(need);
    see_word = __ballot(see);
    word_idx = wi;
  };
  // First needed tile at or after kt (nkt if none).
  auto first_needed = [&](int kt) {
    while (kt < nkt) {
      if ((kt >> 6) != word_idx) load_words(kt >> 6);
      const uint64_t bits = need_word >> (kt & 63);
      if (bits) return kt + (int)__builtin_ctzll(bits);
      kt = (kt | 63) + 1;
    }
    return nkt;
  };
  auto next_tile = [&](int kt) { return a.mask ? first_needed(kt + 1) : kt + 1; };
  // A wave computes a loaded tile only if its own rows see some key of it.
  // Called only for the tile just returned by first_needed / next_tile, so
  // see_word is the word holding kt.
  auto wave_sees = [&](int kt) {
    if (!wave_rows || kt * 64 > klast) return false;
    return !a.mask || ((see_word >> (kt & 63)) & 1);
  };
  // Tile loads go straight to LDS (global_load_lds_dwordx4): wave w's i-th
  // load fills the 1 KB LDS segment 4 i + w, lane l the 16 bytes at 16 l of
  // it.  For K and V a segment is rows 16 i + tid/16 (4 rows of 256 bytes),
  // for the rope part and an fp8 K tile rows 32 i + tid/8 (8 rows of 128
  // bytes).  The LDS swizzle is applied on the global side: the lane that
  // fills LDS chunk c' of a row fetches the chunk that the read swizzle
  // expects there.
  const int row0 = tid >> 4, ch = tid & 15;
  // Rope rows: 128 bytes (bf16; 8 rows per 1 KB segment, 32 per load round)
  // or 64 bytes (fp8 codes; 16 rows per segment, the whole tile in one round).
  constexpr int RRS = RK8 ? 64 : 32;                                   // rope rows per load round
  const int row0r = RK8 ? tid >> 2 : tid >> 3;
  const int chr = RK8 ? tid & 3 : tid & 7;
  const int rch = RK8 ? chr ^ ((row0r >> 2) & 3)                       // fp8 rope: c' = c ^ ((row >> 2) & 3)
                      : chr ^ ((row0r >> 1) & 7);                      // rope: c' = c ^ ((row >> 1) & 7)
  const int vch = (((ch >> 1) ^ vmask(row0)) << 1) | (ch & 1);         // V: 32-byte pieces ^ vmask(row)
  constexpr int KRS = QK8 ? 32 : 16;                                   // K rows per load round
  const int krow = QK8 ? row0r : row0;
  const int kch = QK8 ? rch : ch ^ (row0 & 15);                        // K: c' = c ^ (row & 15)
  // Tile bases are uniform (scalar) pointers; each lane adds one fixed 32-bit
  // byte offset, so the loads use the scalar-base addressing form.
  const int64_t kstr = a.k_st * KGE, vstr = a.v_st * VGE, rstr = a.kr_st * (RK8 ? 1 : 2);  // row strides in bytes
  const unsigned char* kg =
      (const unsigned char*)a.k + ((int64_t)c0 * a.k_st + (int64_t)g * a.k_sh) * KE;
  const unsigned char* vg = (const unsigned char*)(a.v + (int64_t)c0 * a.v_st + (int64_t)g * a.v_sh);
  const unsigned char* rg = DR ? (const unsigned char*)a.kr + (int64_t)c0 * rstr : nullptr;
  const uint32_t koff = (uint32_t)(krow * kstr) + 16u * kch;
  const uint32_t voff = (uint32_t)(row0 * vstr) + 16u * vch;
  const uint32_t roff = DR ? (uint32_t)(row0r * rstr) + 16u * rch : 0u;
  const int wseg = __builtin_amdgcn_readfirstlane(wv) * 1024;
  auto dma = [&](const unsigned char* gp, unsigned char* lp) {
    __builtin_amdgcn_global_load_lds((const void*)gp, (GQAP_LDS void*)lp, 16, 0, 0);
  };
  // Blockwise key scales: lane l of every wave fetches the scale of key l of
  // the tile into the wave's own 256-byte copy.
  auto dma4 = [&](const float* gp, float* lp) {
    __builtin_amdgcn_global_load_lds((const void*)gp, (GQAP_LDS void*)((unsigned char*)lp + (wseg >> 2)), 4, 0, 0);
  };
  // Per-key scales: one per row of a KV head (blockwise fp8 Q.K), or one per
  // rope row shared by every head (fp8 rope keys).
  const int64_t sstr = F8 == 2 ? a.Hk : 1;
  const float* ksg = F8 == 2 ? a.ksc + (int64_t)c0 * a.Hk + g : RK8 ? a.ksc + c0 : nullptr;
  // First byte of key tile kt of K / V.  With PAGED a tile is one page: the
  // 64 x D slab of pool block block_table[b, kt] for KV head g (FlashMLA
  // tensor-shape reference, section 1: tokens 64j .. 64j+63 live in
  // block_table[b, j]).  The table entries are read 64 tiles at a time, one
  // per lane, and picked out with readlane.
  int32_t bt_word = 0;
  int bt_idx = -1;
  auto page_of = [&](int kt) {
    if ((kt >> 6) != bt_idx) {
      bt_idx = kt >> 6;
      const int j = bt_idx * 64 + lane;
      bt_word = j < nkt ? a.bt[(int64_t)b * a.bt_st + j] : 0;
    }
    return __builtin_amdgcn_readlane(bt_word, kt & 63);
  };
  auto tile_k = [&](int kt) -> const unsigned char* {
    if constexpr (PAGED)
      return (const unsigned char*)a.k + ((int64_t)page_of(kt) * a.kv_sb + (int64_t)g * a.kv_sh) * KGE;
    else
      return kg + (int64_t)kt * 64 * kstr;
  };
  auto tile_v = [&](int kt) -> const unsigned char* {
    if constexpr (PAGED)
      return (const unsigned char*)a.v + ((int64_t)page_of(kt) * a.kv_sb + (int64_t)g * a.kv_sh) * VGE;
    else
      return vg + (int64_t)kt * 64 * vstr;
  };
  // The rope keys: one 64 x Dr slab per page with PAGED (one head, shared by
  // every query head), else rows of the token-major rope tensor.
  auto tile_r = [&](int kt) -> const unsigned char* {
    if constexpr (PAGED)
      return (const unsigned char*)a.kr + (int64_t)page_of(kt) * a.kr_sb * 2;
    else
      return rg + (int64_t)kt * 64 * rstr;
  };
  // Rows past the last key read row Lk-1 instead: every key past Lk is
  // causally hidden from every query of the sequence, so its score is
  // replaced by -inf and its probability is exactly 0.
  // fp8 KV pages: lane tid loads the 16 codes at byte 16 c8 of rows row8 and
  // row8 + 32 of the K and of the V page (rows of 128 bytes), into k8r / v8r;
  // stage8 widens them and writes the bf16 tile.
  const int row8 = tid >> 3, c8 = tid & 7;
  const uint32_t koff8 = (uint32_t)(row8 * kstr) + 16u * c8;
  const uint32_t voff8 = (uint32_t)(row8 * vstr) + 16u * c8;
  i32x4 k8r[KV8 ? 2 : 1] = {}, v8r[KV8 ? 2 : 1] = {};
  auto load_tile = [&](int kt, auto bufc) {
    constexpr int BUF = decltype(bufc)::value;
    unsigned char* kd = BUF ? kbuf1 : kbuf0;
    unsigned char* rd = BUF ? rbuf1 : rbuf0;
    unsigned char* vd = BUF ? vbuf1 : vbuf0;
    if constexpr (KSC)
      dma4(ksg + (int64_t)(kt * 64 + min(lane, Lk - 1 - kt * 64)) * sstr, BUF ? sbuf1 : sbuf0);
    const int key0 = kt * 64;
    const unsigned char* kt_k = tile_k(kt);
    const unsigned char* kt_v = tile_v(kt);
    const unsigned char* kt_r = DR ? tile_r(kt) : nullptr;
    if constexpr (KV8) {
      const bool whole = key0 + 64 <= Lk;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int64_t r = whole ? row8 + 32 * i : min(row8 + 32 * i, Lk - 1 - key0);
        k8r[i] = load16(kt_k + r * kstr + 16 * c8);
      }
#pragma unroll
      for (int i = 0; i < RLD; ++i)
        dma(kt_r + (int64_t)(whole ? row0r + 32 * i : min(row0r + 32 * i, Lk - 1 - key0)) * rstr + 16 * rch,
            rd + 4096 * i + wseg);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int64_t r = whole ? row8 + 32 * i : min(row8 + 32 * i, Lk - 1 - key0);
        v8r[i] = load16(kt_v + r * vstr + 16 * c8);
      }
    } else if (key0 + 64 <= Lk) {  // whole tile inside the keys
#pragma unroll
      for (int i = 0; i < KLD; ++i) dma(kt_k + KRS * i * kstr + koff, kd + 4096 * i + wseg);
#pragma unroll
      for (int i = 0; i < RLD; ++i) dma(kt_r + RRS * i * rstr + roff, rd + 4096 * i + wseg);
#pragma unroll
      for (int i = 0; i < VLD; ++i) dma(kt_v + 16 * i * vstr + voff, vd + 4096 * i + wseg);
    } else {
#pragma unroll
      for (int i = 0; i < KLD; ++i)
        dma(kt_k + (int64_t)min(krow + KRS * i, Lk - 1 - key0) * kstr + 16 * kch, kd + 4096 * i + wseg);
#pragma unroll
      for (int i = 0; i < RLD; ++i)
        dma(kt_r + (int64_t)min(row0r + RRS * i, Lk - 1 - key0) * rstr + 16 * rch, rd + 4096 * i + wseg);
#pragma unroll
      for (int i = 0; i < VLD; ++i)
        dma(kt_v + (int64_t)min(row0 + 16 * i, Lk - 1 - key0) * vstr + 16 * vch, vd + 4096 * i + wseg);
    }
    // Keep the loads at the top of the tile so they overlap its math.
    __builtin_amdgcn_sched_barrier(0);
  };
  // fp8 KV pages: widen the codes in k8r / v8r to bf16 and write them where a
  // bf16 tile's loads would have put them: K chunk c of a row (16 bytes) at
  // chunk c ^ (row & 15), V 32-byte piece p at piece p ^ vmask(row).  The
  // buffer written is not read during the current tile; the barrier that ends
  // the tile publishes it.  A wave that computes the tile does this during
  // its P.V steps; when no tile follows, the registers hold stale codes and
  // the buffer they land in is never read again.
  auto stage8 = [&](auto bufc) {
    if constexpr (KV8) {
      constexpr int BUF = decltype(bufc)::value;
      unsigned char* kd = BUF ? kbuf1 : kbuf0;
      unsigned char* vd = BUF ? vbuf1 : vbuf0;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = row8 + 32 * i;
        store16(kd + row * 256 + (((2 * c8) ^ (row & 15)) << 4), fp8x8_to_bf16x8_pk(i32x2{k8r[i][0], k8r[i][1]}));
        store16(kd + row * 256 + (((2 * c8 + 1) ^ (row & 15)) << 4), fp8x8_to_bf16x8_pk(i32x2{k8r[i][2], k8r[i][3]}));
        unsigned char* vp = vd + row * 256 + ((c8 ^ vmask(row)) << 5);
        store16(vp, fp8x8_to_bf16x8_pk(i32x2{v8r[i][0], v8r[i][1]}));
        store16(vp + 16, fp8x8_to_bf16x8_pk(i32x2{v8r[i][2], v8r[i][3]}));
      }
    }
  };
  // Waits for this thread's tile loads; the barrier that follows publishes
  // every thread's.
  auto loads_done = [] { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };

  // Per-lane LDS read offsets; the tile half t, k-step and buffer parts are
  // immediates.  K: chunk (2s + hh) ^ (row & 15) = 2 (s ^ m) + ((hh ^ row) & 1).
  // fp8 K: 16-byte read u = 2 s + e of fp8 step s is chunk 4 s + 2 hh + e,
  // stored at chunk ^ ((row >> 1) & 7).
  int kra[QK8 ? 4 : KSN];
  if constexpr (QK8) {
    const int m = (l32 >> 1) & 7;
#pragma unroll
    for (int u = 0; u < 4; ++u) kra[u] = l32 * 128 + (((4 * (u >> 1) + 2 * hh + (u & 1)) ^ m) << 4);
  } else {
    const int m = (l32 & 15) >> 1;
    const int lo = ((hh ^ l32) & 1) << 4;
#pragma unroll
    for (int s2 = 0; s2 < KSN; ++s2) kra[s2] = l32 * 256 + ((s2 ^ m) << 5) + lo;
  }
  int rra[KSR > 0 ? KSR : 1];
  if constexpr (RK8) {  // 8 codes of k-step s2: chunk s2 of a 64-byte row, half hh of it
    const int m = (l32 >> 2) & 3;
#pragma unroll
    for (int s2 = 0; s2 < KSR; ++s2) rra[s2] = l32 * 64 + ((s2 ^ m) << 4) + 8 * hh;
  } else if constexpr (DR > 0) {
    const int m = (l32 >> 1) & 7;
#pragma unroll
    for (int s2 = 0; s2 < KSR; ++s2) rra[s2] = l32 * 128 + (((2 * s2 + hh) ^ m) << 4);
  }
  // V^T transpose reads: 16-lane group gamma takes d = 32 dt + 16 (gamma & 1) + i
  // from rows kb + li/4, kb = 16 ks + 8 part + 4 hh, so row & 7 = 4 hh + li/4.
  int vra[4];
  {
    const int gam = lane >> 4, li = lane & 15;
    const int row = 4 * hh + (li >> 2);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
      vra[dt] = row * 256 + (((2 * dt + (gam & 1)) ^ vmask(row)) << 5) + 8 * (li & 3);
  }

  float m_run = -INFINITY, l_run = 0.f;  // base-2 scaled max; this lane's half of the row sum
  f32x16_t o[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) o[t] = f32x16_t{};
  const float c = a.scale_log2;

  // compute_tile(kt, BUF, WL, kn): the math of tile kt from buffer BUF; with
  // WL, the loads of tile kn (a whole tile inside the sequence) into the
  // other buffer are issued between its first MFMAs, so that their issue
  // stalls overlap the matrix work instead of preceding it.
  auto compute_tile = [&](int kt, auto bufc, auto wlc, int kn) {
    constexpr int BUF = decltype(bufc)::value;
    constexpr bool WL = decltype(wlc)::value;
    const unsigned char* kb = BUF ? kbuf1 : kbuf0;
    const unsigned char* rb = BUF ? rbuf1 : rbuf0;
    const unsigned char* vb = BUF ? vbuf1 : vbuf0;
    unsigned char* kd = BUF ? kbuf0 : kbuf1;
    unsigned char* rd = BUF ? rbuf0 : rbuf1;
    unsigned char* vd = BUF ? vbuf0 : vbuf1;
    const float* sb = BUF ? sbuf1 : sbuf0;
    float* sd = BUF ? sbuf0 : sbuf1;
    constexpr int NLD = KLD + RLD + VLD + (KSC ? 1 : 0);
    const unsigned char* kt_k = WL ? tile_k(kn) : nullptr;
    const unsigned char* kt_v = WL ? tile_v(kn) : nullptr;
    const unsigned char* kt_r = DR && WL ? tile_r(kn) : nullptr;
    auto issue_load = [&](int i) {
      if constexpr (KV8) {  // whole tile inside the keys: no row clamp
        if (i < KLD)
          k8r[i] = load16(kt_k + 32 * i * kstr + koff8);
        else if (i < KLD + RLD)
          dma(kt_r + 32 * (i - KLD) * rstr + roff, rd + 4096 * (i - KLD) + wseg);
        else
          v8r[i - KLD - RLD] = load16(kt_v + 32 * (i - KLD - RLD) * vstr + voff8);
        return;
      }
      if (i < KLD)
        dma(kt_k + KRS * i * kstr + koff, kd + 4096 * i + wseg);
      else if (i < KLD + RLD)
        dma(kt_r + RRS * (i - KLD) * rstr + roff, rd + 4096 * (i - KLD) + wseg);
      else if (i < KLD + RLD + VLD)
        dma(kt_v + 16 * (i - KLD - RLD) * vstr + voff, vd + 4096 * (i - KLD - RLD) + wseg);
      else if constexpr (KSC)
        dma4(ksg + (int64_t)(kn * 64 + lane) * sstr, sd);
    };
    f32x16_t s[2] = {f32x16_t{}, f32x16_t{}};
    if constexpr (!QK8) {
      // S^T tile t (keys 32t .. 32t+31 of the tile) x 32 queries: 2 NS MFMAs
      // whose K operands are read from LDS PF steps ahead.  With an fp8 cache
      // and a rope part only the nope sum carries k_scale: it is applied
      // before the first rope step of each half.
      constexpr int NS = KSN + KSR;
      constexpr int PF = 8;
      // Matrix step idx of the tile: half t, k-step ss (ss >= KSN: rope).
      // With fp8 rope keys the rope steps of both halves come first.
      auto step_of = [&](int idx, int& t, int& ss) {
        if (RK8 && idx < 2 * KSR) {
          t = idx / KSR;
          ss = KSN + idx % KSR;
        } else if (RK8) {
          t = (idx - 2 * KSR) / KSN;
          ss = (idx - 2 * KSR) % KSN;
        } else {
          t = idx / NS;
          ss = idx % NS;
        }
      };
      auto kfrag = [&](int idx) -> i32x4 {
        int t, ss;
        step_of(idx, t, ss);
        if (ss < KSN) return load16(kb + t * 8192 + kra[ss]);
        if constexpr (RK8) {  // 8 codes -> 8 bf16 values (exact)
          return fp8x8_to_bf16x8_pk(*(const i32x2*)(rb + t * 2048 + rra[ss - KSN]));
        } else {
          return load16(rb + t * 4096 + rra[ss - KSN]);
        }
      };
      // The rope sum of half t times its keys' scales (register j of the
      // half holds key 32 t + 8 (j / 4) + 4 hh + j % 4).
      auto scale_rope = [&](int t) {
        if constexpr (RK8) {
          const float* sp = sb + (wseg >> 4) + 32 * t + 4 * hh;
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const f32x4 w = *(const f32x4*)(sp + 8 * m);
#pragma unroll
            for (int e = 0; e < 4; ++e) s[t][4 * m + e] *= w[e];
          }
        }
      };
      i32x4 kf[PF];
      // Without a rope part the matrix phases run at raised wave priority, so
      // that the SIMD's other wave does not delay a wave that feeds the matrix
      // core (measured: the D = 128 chunked prefill about 8 % faster,
      // block-sparse 1-3 %; with the rope tile neutral to 2 % slower, so left
      // out there).
      if constexpr (DR == 0) __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int i = 0; i < PF; ++i) kf[i] = kfrag(i);
#pragma unroll
      for (int idx = 0; idx < 2 * NS; ++idx) {
        const i32x4 cur = kf[idx % PF];
        if (idx + PF < 2 * NS) kf[idx % PF] = kfrag(idx + PF);
        int t, ss;
        step_of(idx, t, ss);
        if (KV8 && KSR > 0 && ss == KSN) s[t] *= a.qk;
        if (RK8 && ss == 0) scale_rope(t);
        s[t] = mfma32x32x16(__builtin_bit_cast(bf16x8, cur), qop[ss], s[t]);
        if (WL && idx < NLD) issue_load(idx);
      }
      // Issue order: PF reads, then per MFMA one read (and one tile load
      // while any is left).
      __builtin_amdgcn_sched_group_barrier(0x100, PF, 0);
#pragma unroll
      for (int idx = 0; idx < 2 * NS; ++idx) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (idx + PF < 2 * NS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        if (WL && idx < NLD) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
      if constexpr (DR == 0) __builtin_amdgcn_s_setprio(0);
    } else {
      // fp8 nope part: per tile half t two 64-deep fp8 steps, each K operand
      // two 16-byte LDS reads (units 0..7); then the bf16 rope steps (units
      // 8..), after the nope sum of the half has been multiplied by
      // q_scale * k_scale.  Order nope t0, nope t1, rope t0, rope t1, so each
      // multiply waits on a step issued two steps before it.  The tile loads
      // are spread over the NM steps.
      constexpr int NU = 8 + 2 * KSR;
      constexpr int NM = 4 + 2 * KSR;
      constexpr int PF = 8;
      // The nope sum of half t times its scales: per lane (query) and, with
      // blockwise scales, per key (register j holds key 32t + 8(j/4) + 4hh + j%4).
      auto scale_half = [&](int t) {
        if constexpr (F8 == 2) {
          const float* sp = sb + (wseg >> 4) + 32 * t + 4 * hh;
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const f32x4 w = *(const f32x4*)(sp + 8 * m);
#pragma unroll
            for (int e = 0; e < 4; ++e) s[t][4 * m + e] *= qsl * w[e];
          }
        } else {
          s[t] *= qsl;
        }
      };
      auto unit = [&](int u) -> i32x4 {
        if (u < 8) return load16(kb + (u >> 2) * 4096 + kra[u & 3]);
        if constexpr (KSR > 0) {
          const int r = u - 8;
          return load16(rb + (r / KSR) * 4096 + rra[r % KSR]);
        } else {
          return i32x4{};
        }
      };
      i32x4 uf[NU];
#pragma unroll
      for (int u = 0; u < PF; ++u) uf[u] = unit(u);
#pragma unroll
      for (int i = 0; i < NM; ++i) {
        if (i < 4) {
          const int t = i >> 1, st = i & 1;
          const i32x8 ka = __builtin_shufflevector(uf[4 * t + 2 * st], uf[4 * t + 2 * st + 1], 0, 1, 2, 3, 4, 5, 6,
                                                   7);
#pragma unroll
          for (int e = 0; e < 2; ++e)
            if (PF + 2 * i + e < NU) uf[PF + 2 * i + e] = unit(PF + 2 * i + e);
          s[t] = mfma32x32x64_fp8(ka, q8[st], s[t]);
        } else if constexpr (KSR > 0) {
          const int r = i - 4, t = r / KSR;
          if (r % KSR == 0) scale_half(t);
          s[t] = mfma32x32x16(__builtin_bit_cast(bf16x8, uf[8 + r]), qop[r % KSR], s[t]);
        }
        if (WL)
#pragma unroll
          for (int j = i * NLD / NM; j < (i + 1) * NLD / NM; ++j) issue_load(j);
      }
      // Without rope the per-tensor scales are part of the softmax constant.
      if constexpr (KSR == 0 && F8 == 2) {
        scale_half(0);
        scale_half(1);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, PF, 0);
#pragma unroll
      for (int i = 0; i < NM; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i < 4) {
          if (PF + 2 * i < NU) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          if (PF + 2 * i + 1 < NU) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        if (WL)
#pragma unroll
          for (int j = i * NLD / NM; j < (i + 1) * NLD / NM; ++j) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
    }
    // Causal mask by select (only on tiles reaching past the wave's first row).
    if (kt * 64 + 63 > off + r0) {
      const int rel = off + qrow - kt * 64 - hh * 4;  // key offset + hh*4 must stay <= rel
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (32 * t + (j >> 2) * 8 + (j & 3) > rel) s[t][j] = -INFINITY;
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int j = 0; j < 16; ++j) tmax = fmaxf(tmax, s[t][j]);
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, tmax),
                                                       __builtin_bit_cast(uint32_t, tmax), false, false);
      tmax = fmaxf(__builtin_bit_cast(float, (uint32_t)sw[0]), __builtin_bit_cast(float, (uint32_t)sw[1]));
    }
    // The reference point m_run of the exponentials moves only when a score
    // passes it by more than 2^8, so probabilities stay <= 256 (exact range
    // for bf16 and fp32) and the accumulator is rescaled a few times per row
    // instead of on every tile.  The result does not depend on where the
    // reference point sits: out = sum p v / sum p and lse = m_run + log2(sum p).
    const float tm = tmax * c;
    const bool grow = tm > m_run + 8.f;  // also true on the first visible key (m_run = -inf)
    if (__any(grow)) {
      const float m_new = grow ? tm : m_run;
      const float alpha = grow ? fast_exp2(m_run - m_new) : 1.f;  // exp2(-inf) = 0 on the first
      l_run *= alpha;
      m_run = m_new;
#pragma unroll
      for (int t = 0; t < 4; ++t) o[t] *= alpha;
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;  // a row with nothing visible yet
    float psum = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float p = fast_exp2(fmaf(s[t][j], c, -m_use));
        s[t][j] = p;
        psum += p;
      }
    l_run += psum;
    // P^T operands: k-step ks covers keys 16 ks + {4hh .. 4hh+3, 8+4hh .. 8+4hh+3},
    // which are D registers 8 (ks % 2) .. +7 of score tile ks / 2.
    bf16x8 pop[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      i32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        w[e] = (int)pack_bf16x2_hw(s[ks >> 1][8 * (ks & 1) + 2 * e], s[ks >> 1][8 * (ks & 1) + 2 * e + 1]);
      pop[ks] = __builtin_bit_cast(bf16x8, w);
    }
    // O^T[d, q] += V^T P^T, V^T from two transpose reads per k-step, read
    // PV steps ahead of the MFMA that consumes them.
    typedef __attribute__((__vector_size__(8 * sizeof(short)))) short i16x8;
    constexpr int PV = 4;
    auto vfrag = [&](int idx) {
      const int dt = idx >> 2, ks = idx & 3;
      const i16x4 lo = lds_read_tr16(vb + vra[dt] + (16 * ks) * 256);
      const i16x4 hi = lds_read_tr16(vb + vra[dt] + (16 * ks + 8) * 256);
      return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    i16x8 vf[PV];
    if constexpr (DR == 0) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int i = 0; i < PV; ++i) vf[i] = vfrag(i);
    // fp8 pages: the next tile's codes are widened and written between these
    // matrix steps (three conversions and at most one LDS write per step).
    if constexpr (KV8) stage8(std::integral_constant<int, 1 - BUF>{});
#pragma unroll
    for (int idx = 0; idx < 16; ++idx) {
      const i16x8 cur = vf[idx % PV];
      if (idx + PV < 16) vf[idx % PV] = vfrag(idx + PV);
      o[idx >> 2] = mfma32x32x16(__builtin_bit_cast(bf16x8, cur), pop[idx & 3], o[idx >> 2]);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * PV, 0);
#pragma unroll
    for (int idx = 0; idx < 16 - PV; ++idx) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      if constexpr (KV8) {
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
        if (idx < 8) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
      }
    }
    __builtin_amdgcn_sched_group_barrier(0x008, PV, 0);
    if constexpr (DR == 0) __builtin_amdgcn_s_setprio(0);
  };

  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  int kt = a.mask ? first_needed(kt_begin) : kt_begin;
  if (kt < kt_end) {
    load_tile(kt, B0{});
    stage8(B0{});
  }
  loads_done();
  __syncthreads();
  using WL0 = std::integral_constant<bool, false>;
  using WL1 = std::integral_constant<bool, true>;
  // One tile: the loads of the next needed tile kn go into the other buffer,
  // interleaved with this tile's matrix work when this wave computes and kn
  // lies wholly inside the sequence, else up front.
  auto step = [&](int kt, bool sees, int kn, auto bufc, auto nbufc) {
    const bool more = kn < kt_end;
    const bool inside = more && kn * 64 + 64 <= Lk;
    if (sees && inside) {
      compute_tile(kt, bufc, WL1{}, kn);  // with fp8 pages, stages kn during its P.V steps
    } else {
      if (more) load_tile(kn, nbufc);
      if (sees)
        compute_tile(kt, bufc, WL0{}, kn);
      else if (more)
        stage8(nbufc);
    }
    loads_done();
    __syncthreads();
  };
  // Two tiles per trip so the LDS buffer index is static.  wave_sees(kt) is
  // read before next_tile() may move the bit words on to the next 64 tiles.
  // A buffer is refilled only after the barrier that ends the reads of it.
  while (kt < kt_end) {
    bool sees = wave_sees(kt);
    int kn = next_tile(kt);
    step(kt, sees, kn, B0{}, B1{});
    kt = kn;
    if (kt >= kt_end) break;
    sees = wave_sees(kt);
    kn = next_tile(kt);
    step(kt, sees, kn, B1{}, B0{});
    kt = kn;
  }

  // Epilogue: combine the two halves of each row sum, normalise, store.
  if (!wave_rows) return;
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, l_run),
                                                     __builtin_bit_cast(uint32_t, l_run), false, false);
    l_run = __builtin_bit_cast(float, (uint32_t)sw[0]) + __builtin_bit_cast(float, (uint32_t)sw[1]);
  }
  if (qrow >= L) return;
  const float inv = l_run > 0.f ? (KV8 ? a.v_scale : 1.f) / l_run : 0.f;
  if (a.nsplit > 1) {  // partial of this key range; prefill_merge writes the output
    const int64_t prow = ((int64_t)sp * a.T + c0 + qrow) * a.Hq + h;
    float* wp = a.ws_o + prow * DV;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int J = 0; J < 4; ++J) {
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = o[dt][4 * J + e] * inv;
        *(f32x4*)(wp + 32 * dt + 8 * J + 4 * hh) = v;
      }
    if (hh == 0) a.ws_lse[prow] = l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
    return;
  }
  uint16_t* op = a.out + (int64_t)(c0 + qrow) * a.o_st + (int64_t)h * a.o_sh;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      // D registers 4J..4J+3 hold d = 32 dt + 8 J + 4 hh + 0..3
      const int d = 32 * dt + 8 * J + 4 * hh;
      i32x2 w;
      w[0] = (int)pack_bf16x2_hw(o[dt][4 * J] * inv, o[dt][4 * J + 1] * inv);
      w[1] = (int)pack_bf16x2_hw(o[dt][4 * J + 2] * inv, o[dt][4 * J + 3] * inv);
      *(i32x2*)(op + d) = w;
    }
  if (a.lse && hh == 0)
    a.lse[(int64_t)(c0 + qrow) * a.Hq + h] = l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
}


// Merge of the key-axis splits of one (row, head): with w_s = exp(lse_s -
// max lse), out = sum_s w_s o_s / sum_s w_s and lse = max + log(sum_s w_s);
// a row that no split saw any key for gets 0 / -inf.  One wave merges R
// consecutive (row, head) pairs, two output columns per lane;
// all their LSEs and partial rows (up to four splits) and the sequence
// bounds are requested before any is used, so a wave costs one memory round
// trip.  Rows that are not outputs (past cu[B], or past the planned length
// of their sequence) are skipped, as the attention kernel skips them.
struct MergeArgs {
  const float* ws_o;
  const float* ws_lse;
  const int32_t* cu;
  const int32_t* kvlens;  // chunked prefill: keys per sequence, else null
  uint16_t* out;
  float* lse;
  int64_t o_st, o_sh;
  int32_t T, Hq, B, nsplit, max_len, max_kv;
};

template <int R>
__global__ __launch_bounds__(256) void prefill_merge(MergeArgs a) {
  constexpr int NU = 4;  // splits merged in the single round trip; more take a loop
  const int lane = threadIdx.x & 63;
  const int64_t nrh = (int64_t)a.T * a.Hq;
  const int64_t rh0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * R;
  if (rh0 >= nrh) return;
  // The LSEs and partial rows of the pairs are requested first (every slot
  // below T * Hq lies inside the workspace; slots of rows that are not
  // outputs are read but never used), together with the sequence bounds:
  // with B < 64 lane l holds cu[l] (l <= B) and kvlens[l] and a row's
  // sequence is found by a ballot; larger batches take a binary search.
  const int64_t sstride = nrh;
  float ls[R][NU];
  f32x2 v[R][NU];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int s = 0; s < NU; ++s) {
      const int64_t rh = rh0 + r;
      const bool ld = rh < nrh && s < a.nsplit;
      ls[r][s] = ld ? a.ws_lse[s * sstride + rh] : -INFINITY;
      v[r][s] = ld ? *(const f32x2*)(a.ws_o + (s * sstride + rh) * 128 + 2 * lane) : f32x2{0.f, 0.f};
    }
  const bool small = a.B < 64;
  int cu_l = 0, kv_l = 0;
  if (small) {
    if (lane <= a.B) cu_l = a.cu[lane];
    if (a.kvlens && lane < a.B) kv_l = a.kvlens[lane];
  }
  const int cu_end = small ? __shfl(cu_l, a.B) : a.cu[a.B];
  bool live[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t rh = rh0 + r;
    const int row = rh < nrh ? (int)(rh / a.Hq) : cu_end;
    int c0, c1, kl = 0;
    if (small) {
      const int b = __popcll(__ballot(lane <= a.B && cu_l <= row)) - 1;  // cu is non-decreasing
      c0 = __shfl(cu_l, b);
      c1 = __shfl(cu_l, b + 1);
      kl = __shfl(kv_l, b);
    } else {
      int lo = 0, hi = a.B;  // the sequence b with cu[b] <= row < cu[b + 1]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (a.cu[mid] <= row) lo = mid; else hi = mid;
      }
      c0 = a.cu[lo];
      c1 = a.cu[lo + 1];
      if (a.kvlens) kl = a.kvlens[lo];
    }
    // (a chunk outside the capacity was cleared by the attention kernel)
    live[r] = row < cu_end && row - c0 < a.max_len && (!a.kvlens || (kl <= a.max_kv && kl >= c1 - c0));
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (!live[r]) continue;
    const int64_t rh = rh0 + r;
    float M = -INFINITY;
#pragma unroll
    for (int s = 0; s < NU; ++s) M = fmaxf(M, ls[r][s]);
    for (int s = NU; s < a.nsplit; ++s) M = fmaxf(M, a.ws_lse[s * sstride + rh]);
    float den = 0.f, acc0 = 0.f, acc1 = 0.f;
    if (M > -INFINITY) {
#pragma unroll
      for (int s = 0; s < NU; ++s) {
        const float wgt = ls[r][s] == -INFINITY ? 0.f : expf(ls[r][s] - M);
        den += wgt;
        acc0 += wgt * v[r][s][0];
        acc1 += wgt * v[r][s][1];
      }
      for (int s = NU; s < a.nsplit; ++s) {
        const float lsx = a.ws_lse[s * sstride + rh];
        if (lsx == -INFINITY) continue;
        const float wgt = expf(lsx - M);
        const f32x2 vx = *(const f32x2*)(a.ws_o + (s * sstride + rh) * 128 + 2 * lane);
        den += wgt;
        acc0 += wgt * vx[0];
        acc1 += wgt * vx[1];
      }
    }
    const int row = (int)(rh / a.Hq);
    const int h = (int)(rh - (int64_t)row * a.Hq);
    const float inv = den > 0.f ? 1.f / den : 0.f;
    *(uint32_t*)(a.out + (int64_t)row * a.o_st + (int64_t)h * a.o_sh + 2 * lane) =
        pack_bf16x2_hw(acc0 * inv, acc1 * inv);
    if (a.lse && lane == 0) a.lse[rh] = den > 0.f ? M + logf(den) : -INFINITY;
  }
}

// Append a chunk's keys and values to the paged cache (FlashMLA tensor-shape
// reference, section 4, "Prefill to Cache Mapping": token p of a sequence is
// row p % 64 of block block_table[b, p / 64]).  The chunk of sequence b is
// the last q_len of its kv_len keys, so its token i lands at p = kv_len -
// q_len + i.  One thread per 16-byte piece of a (token, KV head) row.
struct AppendArgs {
  const uint16_t* k_new;
  const uint16_t* v_new;
  uint16_t* k_pool;
  uint16_t* v_pool;
  const int32_t* bt;
  const int32_t* cu;
  const int32_t* kvlens;
  const uint16_t* kr_new;  // MLA: [T, 1, 64] rope keys, or null
  uint16_t* kr_pool;       // MLA: [NB, 1, 64, 64], or null
  int64_t new_st, new_sh, kv_sb, kv_sh, bt_st, kr_new_st, kr_sb;
  int64_t rows;     // T * Hk
  int32_t B, Hk, max_kv;
  float k_scale, v_scale;  // fp8 pools: a code c stands for e4m3fn(c) * scale
};

// Code of x / scale in OCP e4m3fn for two values at a time, into byte pair
// HI of w.  The quotient is the correctly rounded float32 one; magnitudes
// past the largest finite value 448 saturate to it (the format has no
// infinity; NaN stays NaN and gives a NaN code), and the hardware conversion
// rounds to the nearest value, ties to even.
__device__ __forceinline__ float sat_e4m3(float y) { return fabsf(y) > 448.f ? copysignf(448.f, y) : y; }
template <bool HI>
__device__ __forceinline__ int quant_pair(uint32_t bf2, float scale, int w) {
  const float x0 = dev::bf16_to_f32((uint16_t)(bf2 & 0xffffu));
  const float x1 = dev::bf16_to_f32((uint16_t)(bf2 >> 16));
  return __builtin_amdgcn_cvt_pk_fp8_f32(sat_e4m3(__fdiv_rn(x0, scale)), sat_e4m3(__fdiv_rn(x1, scale)), w, HI);
}

template <bool FP8>
__global__ __launch_bounds__(256) void append_kv(AppendArgs a) {
  constexpr int D = 128;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = gid >> 4;
  const int piece = (int)(gid & 15);
  if (row >= a.rows) return;
  const int t = (int)(row / a.Hk), g = (int)(row - (int64_t)t * a.Hk);
  if (t >= a.cu[a.B]) return;  // rows past the last chunk
  int lo = 0, hi = a.B;        // the sequence b with cu[b] <= t < cu[b + 1]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.cu[mid] <= t) lo = mid; else hi = mid;
  }
  const int b = lo;
  const int kl = a.kvlens[b], ql = a.cu[b + 1] - a.cu[b];
  if (kl > a.max_kv || kl < ql) return;  // a chunk outside the plan's capacity writes nothing
  const int p = kl - ql + (t - a.cu[b]);
  const int64_t page = a.bt[(int64_t)b * a.bt_st + (p >> 6)];
  const int64_t dst = page * a.kv_sb + (int64_t)g * a.kv_sh + (int64_t)(p & 63) * D + 8 * piece;
  const int64_t src = (int64_t)t * a.new_st + (int64_t)g * a.new_sh + 8 * piece;
  if constexpr (FP8) {  // 8 values -> 8 code bytes; dst counts bytes
    const dev::i32x4 kx = dev::load16(a.k_new + src), vx = dev::load16(a.v_new + src);
    dev::i32x2 kc, vc;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      kc[e] = quant_pair<true>((uint32_t)kx[2 * e + 1], a.k_scale, quant_pair<false>((uint32_t)kx[2 * e], a.k_scale, 0));
      vc[e] = quant_pair<true>((uint32_t)vx[2 * e + 1], a.v_scale, quant_pair<false>((uint32_t)vx[2 * e], a.v_scale, 0));
    }
    *(dev::i32x2*)((unsigned char*)a.k_pool + dst) = kc;
    *(dev::i32x2*)((unsigned char*)a.v_pool + dst) = vc;
  } else {
    dev::store16(a.k_pool + dst, dev::load16(a.k_new + src));
    dev::store16(a.v_pool + dst, dev::load16(a.v_new + src));
  }
  if (a.kr_pool && g == 0 && piece < 8)  // the 128-byte rope row, once per token
    dev::store16(a.kr_pool + page * a.kr_sb + (int64_t)(p & 63) * 64 + 8 * piece,
                 dev::load16(a.kr_new + (int64_t)t * a.kr_new_st + 8 * piece));
}

static bool misaligned16(const void* p) { return ((uintptr_t)p) & 15; }

// Key-axis splits: the workspace holds the partial outputs [nsplit][T][Hq][128]
// fp32, then the partial LSEs [nsplit][T][Hq].
static gqap_status split_setup(int32_t nsplit, int32_t T, int32_t Hq, uint64_t need, void* workspace,
                               uint64_t workspace_bytes, PrefillArgs* a) {
  a->nsplit = nsplit > 1 ? nsplit : 1;
  a->T = T;
  if (a->nsplit == 1) return GQAP_OK;
  if (!workspace || workspace_bytes < need)
    return fail(GQAP_ERR_INVALID_ARGUMENT, "this plan splits the key axis %d ways and needs a workspace of %llu bytes",
                nsplit, (unsigned long long)need);
  if (misaligned16(workspace)) return fail(GQAP_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
  a->ws_o = (float*)workspace;
  a->ws_lse = (float*)((unsigned char*)workspace + (uint64_t)nsplit * (uint64_t)T * (uint64_t)Hq * 128u * 4u);
  return GQAP_OK;
}

// Workgroups of a prefill launch: Hq / hpw per (sequence, query tile) item
// and split.  Up to 64 sequences the kernel ranks the items that exist, so
// the grid needs no more items than the rows can fill: a sequence of L rows
// has ceil(L / QT) tiles, at most (L + QT - 1) / QT, and the rows of all
// sequences are at most T, so sum_b ceil(L_b / QT) <= (T + B (QT - 1)) / QT.
// Every item past that bound would only return (each costs its compute unit
// slot a couple of microseconds: the read of the sequence lengths).
static dim3 prefill_grid(int32_t B, int32_t Hq, int32_t hpw, int32_t q_tiles, int32_t nsplit, int64_t T) {
  const int64_t QT = 128 / hpw;
  int64_t items = (int64_t)B * q_tiles;
  if (B <= 64) items = std::min<int64_t>(items, std::max<int64_t>(B ? 1 : 0, (T + (int64_t)B * (QT - 1)) / QT));
  return dim3((unsigned)((int64_t)(Hq / hpw) * items * nsplit));
}

static gqap_status launch_merge(const PrefillArgs& a, int32_t max_len, hipStream_t st) {
  if (a.nsplit <= 1) return GQAP_OK;
  MergeArgs m{};
  m.ws_o = a.ws_o;
  m.ws_lse = a.ws_lse;
  m.cu = a.cu;
  m.out = a.out;
  m.lse = a.lse;
  m.o_st = a.o_st;
  m.o_sh = a.o_sh;
  m.T = a.T;
  m.Hq = a.Hq;
  m.B = a.B;
  m.nsplit = a.nsplit;
  m.max_len = max_len;
  m.kvlens = a.kvlens;
  m.max_kv = a.max_kv;
  // Pairs per wave: a second pair amortises a wave's start and its sequence
  // lookup, but the merge is one memory round trip per wave, so a small grid
  // keeps one pair per wave to have more waves in flight.  Measured per merge
  // (bf16 out, 128 columns): 8192 pairs, 4 splits: 6.8 / 6.9 / 8.0 us with
  // 1 / 2 / 4 pairs per wave; 32768 pairs, 2 splits: 14.3 / 14.2 / 15.7;
  // 131072 pairs, 2 splits: 51.5 / 48.1 / 50.9.
  const int64_t nrh = (int64_t)a.T * a.Hq;
  const int R = nrh >= 2 * 8192 ? 2 : 1;
  const int64_t blocks = (nrh + 4 * R - 1) / (4 * R);
  if (blocks == 0) return GQAP_OK;
  if (R == 2)
    hipLaunchKernelGGL(prefill_merge<2>, dim3((unsigned)blocks), dim3(256), 0, st, m);
  else
    hipLaunchKernelGGL(prefill_merge<1>, dim3((unsigned)blocks), dim3(256), 0, st, m);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(GQAP_ERR_HIP, "split merge launch: %s", hipGetErrorString(e));
  return GQAP_OK;
}

}  // namespace gqap

using namespace gqap;

// Fields shared by the bf16 and fp8 ragged launches.
static PrefillArgs ragged_args(const gqap_prefill_plan_t* plan, const int32_t* cu_seqlens,
                               const uint8_t* block_mask, void* out, float* lse) {
  const gqap_prefill_desc_t& d = plan->desc;
  PrefillArgs a{};
  a.cu = cu_seqlens;
  a.mask = d.has_block_mask ? block_mask : nullptr;
  a.out = (uint16_t*)out;
  a.lse = lse;
  a.q_st = d.q_stride_token;
  a.q_sh = d.q_stride_head;
  a.k_st = d.k_stride_token;
  a.k_sh = d.k_stride_head;
  a.v_st = d.v_stride_token;
  a.v_sh = d.v_stride_head;
  a.kr_st = d.kr_stride_token;
  a.o_st = d.out_stride_token;
  a.o_sh = d.out_stride_head;
  a.B = d.batch;
  a.Hq = d.num_q_heads;
  a.Hk = d.num_kv_heads;
  a.ratio = plan->ratio;
  a.q_tiles = plan->q_tiles;
  a.hpw = 128 / plan->q_tile_rows;
  a.mask_nb = d.mask_blocks;
  a.max_len = d.max_seq_len;
  return a;
}

extern "C" gqap_status gqap_prefill(const gqap_prefill_plan_t* plan, const void* q, const void* k, const void* v,
                                    const void* k_rope, const int32_t* cu_seqlens, const uint8_t* block_mask,
                                    float scale, void* out, float* lse, void* workspace, uint64_t workspace_bytes,
                                    void* stream) {
  if (!plan || plan->magic != GQAP_PLAN_MAGIC) return fail(GQAP_ERR_INVALID_ARGUMENT, "invalid prefill plan");
  const gqap_prefill_desc_t& d = plan->desc;
  if (d.dtype != GQAP_BF16) return fail(GQAP_ERR_DTYPE, "gqap_prefill takes a bf16 plan (fp8: gqap_prefill_fp8)");
  if (d.batch == 0 || plan->q_tiles == 0) return GQAP_OK;
  if (!q || !k || !v || !cu_seqlens || !out) return fail(GQAP_ERR_INVALID_ARGUMENT, "null device pointer");
  if (d.head_dim_rope && !k_rope) return fail(GQAP_ERR_INVALID_ARGUMENT, "k_rope is required when head_dim_rope > 0");
  if (!d.head_dim_rope && k_rope) return fail(GQAP_ERR_INVALID_ARGUMENT, "k_rope given but head_dim_rope == 0");
  if (d.has_block_mask && !block_mask) return fail(GQAP_ERR_INVALID_ARGUMENT, "block mask declared but null");
  if (misaligned16(q) || misaligned16(k) || misaligned16(v) || misaligned16(out) ||
      (k_rope && misaligned16(k_rope)) || ((uintptr_t)cu_seqlens & 3) || (lse && ((uintptr_t)lse & 3)))
    return fail(GQAP_ERR_INVALID_ARGUMENT, "device pointers must be 16-byte aligned (cu_seqlens, lse 4-byte)");
  if (!std::isfinite(scale)) return fail(GQAP_ERR_INVALID_ARGUMENT, "scale must be finite");
  PrefillArgs a = ragged_args(plan, cu_seqlens, block_mask, out, lse);
  const gqap_status ss =
      split_setup((int32_t)plan->num_splits, d.total_tokens, d.num_q_heads, plan->workspace_bytes, workspace,
                  workspace_bytes, &a);
  if (ss != GQAP_OK) return ss;
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.kr = (const uint16_t*)k_rope;
  a.scale_log2 = scale * dev::kLog2e;
  const dim3 grid = prefill_grid(d.batch, d.num_q_heads, a.hpw, plan->q_tiles, a.nsplit, d.total_tokens);
  hipStream_t st = (hipStream_t)stream;
  if (d.head_dim_rope == 64)
    hipLaunchKernelGGL((prefill_fwd<64, false, 0>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((prefill_fwd<0, false, 0>), grid, dim3(256), 0, st, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(GQAP_ERR_HIP, "prefill launch: %s", hipGetErrorString(e));
  return launch_merge(a, d.max_seq_len, st);
}

extern "C" gqap_status gqap_prefill_rope_fp8(const gqap_prefill_plan_t* plan, const void* q, const void* k,
                                             const void* v, const void* k_rope, const float* k_rope_scales,
                                             const int32_t* cu_seqlens, const uint8_t* block_mask, float scale,
                                             void* out, float* lse, void* workspace, uint64_t workspace_bytes,
                                             void* stream) {
  if (!plan || plan->magic != GQAP_PLAN_MAGIC) return fail(GQAP_ERR_INVALID_ARGUMENT, "invalid prefill plan");
  const gqap_prefill_desc_t& d = plan->desc;
  if (d.dtype != GQAP_BF16)
    return fail(GQAP_ERR_DTYPE, "gqap_prefill_rope_fp8 takes a bf16 plan (q, k and v are bf16)");
  if (d.head_dim_rope != 64)
    return fail(GQAP_ERR_INVALID_ARGUMENT, "gqap_prefill_rope_fp8 needs the MLA split head (head_dim_rope 64)");
  if (d.kr_stride_token % 16 || d.kr_stride_token < 64)
    return fail(GQAP_ERR_INVALID_ARGUMENT,
                "the fp8 rope rows need a token stride of at least 64 bytes, a multiple of 16 (got %lld)",
                (long long)d.kr_stride_token);
  if (!std::isfinite(scale)) return fail(GQAP_ERR_INVALID_ARGUMENT, "scale must be finite");
  if (d.batch == 0 || plan->q_tiles == 0) return GQAP_OK;
  if (!q || !k || !v || !k_rope || !k_rope_scales || !cu_seqlens || !out)
    return fail(GQAP_ERR_INVALID_ARGUMENT, "null device pointer");
  if (d.has_block_mask && !block_mask) return fail(GQAP_ERR_INVALID_ARGUMENT, "block mask declared but null");
  if (misaligned16(q) || misaligned16(k) || misaligned16(v) || misaligned16(out) || misaligned16(k_rope) ||
      ((uintptr_t)k_rope_scales & 3) || ((uintptr_t)cu_seqlens & 3) || (lse && ((uintptr_t)lse & 3)))
    return fail(GQAP_ERR_INVALID_ARGUMENT,
                "device pointers must be 16-byte aligned (k_rope_scales, cu_seqlens, lse 4-byte)");
  PrefillArgs a = ragged_args(plan, cu_seqlens, block_mask, out, lse);
  const gqap_status ss =
      split_setup((int32_t)plan->num_splits, d.total_tokens, d.num_q_heads, plan->workspace_bytes, workspace,
                  workspace_bytes, &a);
  if (ss != GQAP_OK) return ss;
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.kr = (const uint16_t*)k_rope;  // e4m3fn codes; the kernel reads bytes
  a.ksc = k_rope_scales;
  a.scale_log2 = scale * dev::kLog2e;
  const dim3 grid = prefill_grid(d.batch, d.num_q_heads, a.hpw, plan->q_tiles, a.nsplit, d.total_tokens);
  hipStream_t st = (hipStream_t)stream;
  hipLaunchKernelGGL((prefill_fwd<64, false, 4>), grid, dim3(256), 0, st, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(GQAP_ERR_HIP, "fp8-rope prefill launch: %s", hipGetErrorString(e));
  return launch_merge(a, d.max_seq_len, st);
}

// Checks and argument set-up shared by the two fp8 entry points.
static gqap_status fp8_args(const gqap_prefill_plan_t* plan, const void* q_nope, const void* q_rope, const void* k,
                            const void* v, const void* k_rope, const int32_t* cu_seqlens, const uint8_t* block_mask,
                            float scale, void* out, float* lse, PrefillArgs* a) {
  if (!plan || plan->magic != GQAP_PLAN_MAGIC) return fail(GQAP_ERR_INVALID_ARGUMENT, "invalid prefill plan");
  const gqap_prefill_desc_t& d = plan->desc;
  if (d.dtype != GQAP_FP8_E4M3FN)
    return fail(GQAP_ERR_DTYPE, "the fp8 prefill takes a plan with dtype GQAP_FP8_E4M3FN");
  if (!std::isfinite(scale)) return fail(GQAP_ERR_INVALID_ARGUMENT, "scale must be finite");
  if (d.batch == 0 || plan->q_tiles == 0) return GQAP_OK;
  if (!q_nope || !k || !v || !cu_seqlens || !out) return fail(GQAP_ERR_INVALID_ARGUMENT, "null device pointer");
  if (d.head_dim_rope && (!k_rope || !q_rope))
    return fail(GQAP_ERR_INVALID_ARGUMENT, "q_rope and k_rope are required when head_dim_rope > 0");
  if (!d.head_dim_rope && (k_rope || q_rope))
    return fail(GQAP_ERR_INVALID_ARGUMENT, "rope tensors given but head_dim_rope == 0");
  if (d.has_block_mask && !block_mask) return fail(GQAP_ERR_INVALID_ARGUMENT, "block mask declared but null");
  if (misaligned16(q_nope) || misaligned16(k) || misaligned16(v) || misaligned16(out) ||
      (k_rope && misaligned16(k_rope)) || (q_rope && misaligned16(q_rope)) || ((uintptr_t)cu_seqlens & 3) ||
      (lse && ((uintptr_t)lse & 3)))
    return fail(GQAP_ERR_INVALID_ARGUMENT, "device pointers must be 16-byte aligned (cu_seqlens, lse 4-byte)");
  *a = ragged_args(plan, cu_seqlens, block_mask, out, lse);
  a->q = (const uint16_t*)q_nope;
  a->k = (const uint16_t*)k;
  a->v = (const uint16_t*)v;
  a->kr = (const uint16_t*)k_rope;
  a->qr = (const uint16_t*)q_rope;
  a->qr_st = d.qr_stride_token;
  a->qr_sh = d.qr_stride_head;
  a->scale_log2 = scale * dev::kLog2e;
  return GQAP_OK;
}

template <int F8>
static gqap_status launch_fp8(const gqap_prefill_plan_t* plan, PrefillArgs& a, void* workspace,
                              uint64_t workspace_bytes, void* stream) {
  const gqap_prefill_desc_t& d = plan->desc;
  const gqap_status ss = split_setup((int32_t)plan->num_splits, d.total_tokens, d.num_q_heads, plan->workspace_bytes,
                                     workspace, workspace_bytes, &a);
  if (ss != GQAP_OK) return ss;
  const dim3 grid = prefill_grid(d.batch, d.num_q_heads, a.hpw, plan->q_tiles, a.nsplit, d.total_tokens);
  hipStream_t st = (hipStream_t)stream;
  if (d.head_dim_rope == 64)
    hipLaunchKernelGGL((prefill_fwd<64, false, F8>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((prefill_fwd<0, false, F8>), grid, dim3(256), 0, st, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(GQAP_ERR_HIP, "fp8 prefill launch: %s", hipGetErrorString(e));
  return launch_merge(a, d.max_seq_len, st);
}

extern "C" gqap_status gqap_prefill_fp8(const gqap_prefill_plan_t* plan, const void* q_nope, const void* q_rope,
                                        const void* k, const void* v, const void* k_rope,
                                        const int32_t* cu_seqlens, const uint8_t* block_mask, float scale,
                                        float q_scale, float k_scale, void* out, float* lse, void* workspace,
                                        uint64_t workspace_bytes, void* stream) {
  if (!std::isfinite(q_scale) || !std::isfinite(k_scale))
    return fail(GQAP_ERR_INVALID_ARGUMENT, "scale, q_scale and k_scale must be finite");
  PrefillArgs a{};
  const gqap_status s = fp8_args(plan, q_nope, q_rope, k, v, k_rope, cu_seqlens, block_mask, scale, out, lse, &a);
  if (s != GQAP_OK || plan->desc.batch == 0 || plan->q_tiles == 0) return s;
  // With the rope part the nope sum is scaled inside the kernel; without it
  // the whole score is the nope sum and the scales join the softmax constant.
  a.qk = q_scale * k_scale;
  if (!plan->desc.head_dim_rope) a.scale_log2 *= a.qk;
  return launch_fp8<1>(plan, a, workspace, workspace_bytes, stream);
}

extern "C" gqap_status gqap_prefill_fp8_blockwise(const gqap_prefill_plan_t* plan, const void* q_nope,
                                                  const void* q_rope, const void* k, const void* v,
                                                  const void* k_rope, const int32_t* cu_seqlens,
                                                  const uint8_t* block_mask, float scale, const float* q_scales,
                                                  const float* k_scales, void* out, float* lse, void* workspace,
                                                  uint64_t workspace_bytes, void* stream) {
  PrefillArgs a{};
  const gqap_status s = fp8_args(plan, q_nope, q_rope, k, v, k_rope, cu_seqlens, block_mask, scale, out, lse, &a);
  if (s != GQAP_OK || plan->desc.batch == 0 || plan->q_tiles == 0) return s;
  if (!q_scales || !k_scales) return fail(GQAP_ERR_INVALID_ARGUMENT, "q_scales and k_scales are required");
  if (((uintptr_t)q_scales & 3) || ((uintptr_t)k_scales & 3))
    return fail(GQAP_ERR_INVALID_ARGUMENT, "q_scales and k_scales must be 4-byte aligned");
  a.qsc = q_scales;
  a.ksc = k_scales;
  return launch_fp8<2>(plan, a, workspace, workspace_bytes, stream);
}

// The cache's storage: bf16 (kv_dtype 0 or GQAP_BF16) or fp8 e4m3fn codes.
static bool chunk_fp8_cache(const gqap_chunk_desc_t& d) { return d.kv_dtype == GQAP_FP8_E4M3FN; }

static gqap_status append_common(const gqap_chunk_plan_t* plan, const void* k_new, const void* v_new,
                                 const void* k_rope_new, void* k_pool, void* v_pool, void* kr_pool,
                                 const int32_t* block_table, const int32_t* cu_seqlens_q, const int32_t* kv_lens,
                                 bool fp8, float k_scale, float v_scale, void* stream) {
  if (!plan || plan->magic != GQAP_PLAN_MAGIC) return fail(GQAP_ERR_INVALID_ARGUMENT, "invalid chunk plan");
  const gqap_chunk_desc_t& d = plan->desc;
  if (chunk_fp8_cache(d) != fp8)
    return fail(GQAP_ERR_DTYPE, fp8 ? "gqap_append_kv_fp8 needs a plan with kv_dtype GQAP_FP8_E4M3FN"
                                    : "this plan has an fp8 cache: append with gqap_append_kv_fp8");
  if (fp8 && !(std::isfinite(k_scale) && k_scale > 0.f && std::isfinite(v_scale) && v_scale > 0.f))
    return fail(GQAP_ERR_INVALID_ARGUMENT, "k_scale and v_scale must be finite and > 0");
  if (d.batch == 0 || d.total_q_tokens == 0) return GQAP_OK;
  if (!k_new || !v_new || !k_pool || !v_pool || !block_table || !cu_seqlens_q || !kv_lens)
    return fail(GQAP_ERR_INVALID_ARGUMENT, "null device pointer");
  if (d.head_dim_rope && (!k_rope_new || !kr_pool))
    return fail(GQAP_ERR_INVALID_ARGUMENT, "k_rope_new and kr_pool are required when head_dim_rope > 0");
  if (!d.head_dim_rope && (k_rope_new || kr_pool))
    return fail(GQAP_ERR_INVALID_ARGUMENT, "rope tensors given but head_dim_rope == 0");
  if (misaligned16(k_new) || misaligned16(v_new) || misaligned16(k_pool) || misaligned16(v_pool) ||
      (kr_pool && (misaligned16(kr_pool) || misaligned16(k_rope_new))) || ((uintptr_t)block_table & 3) ||
      ((uintptr_t)cu_seqlens_q & 3) || ((uintptr_t)kv_lens & 3))
    return fail(GQAP_ERR_INVALID_ARGUMENT, "device pointers must be 16-byte aligned (index arrays 4-byte)");
  AppendArgs a{};
  a.k_new = (const uint16_t*)k_new;
  a.v_new = (const uint16_t*)v_new;
  a.k_pool = (uint16_t*)k_pool;
  a.v_pool = (uint16_t*)v_pool;
  a.bt = block_table;
  a.cu = cu_seqlens_q;
  a.kvlens = kv_lens;
  a.kr_new = (const uint16_t*)k_rope_new;
  a.kr_pool = (uint16_t*)kr_pool;
  a.kr_new_st = d.kr_new_stride_token;
  a.kr_sb = d.kr_stride_block;
  a.new_st = d.new_stride_token;
  a.new_sh = d.new_stride_head;
  a.kv_sb = d.kv_stride_block;
  a.kv_sh = d.kv_stride_head;
  a.bt_st = d.block_table_stride;
  a.rows = (int64_t)d.total_q_tokens * d.num_kv_heads;
  a.B = d.batch;
  a.Hk = d.num_kv_heads;
  a.max_kv = d.max_kv_len;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  if (a.rows * 16 > kMaxLaunchItems) return fail(GQAP_ERR_UNSUPPORTED, "chunk too large for one append launch");
  const int64_t blocks = (a.rows * 16 + 255) / 256;
  if (fp8)
    hipLaunchKernelGGL(append_kv<true>, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, a);
  else
    hipLaunchKernelGGL(append_kv<false>, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(GQAP_ERR_HIP, "append launch: %s", hipGetErrorString(e));
  return GQAP_OK;
}

extern "C" gqap_status gqap_append_kv(const gqap_chunk_plan_t* plan, const void* k_new, const void* v_new,
                                      const void* k_rope_new, void* k_pool, void* v_pool, void* kr_pool,
                                      const int32_t* block_table, const int32_t* cu_seqlens_q,
                                      const int32_t* kv_lens, void* stream) {
  return append_common(plan, k_new, v_new, k_rope_new, k_pool, v_pool, kr_pool, block_table, cu_seqlens_q, kv_lens,
                       false, 1.f, 1.f, stream);
}

extern "C" gqap_status gqap_append_kv_fp8(const gqap_chunk_plan_t* plan, const void* k_new, const void* v_new,
                                          const void* k_rope_new, void* k_pool, void* v_pool, void* kr_pool,
                                          const int32_t* block_table, const int32_t* cu_seqlens_q,
                                          const int32_t* kv_lens, float k_scale, float v_scale, void* stream) {
  return append_common(plan, k_new, v_new, k_rope_new, k_pool, v_pool, kr_pool, block_table, cu_seqlens_q, kv_lens,
                       true, k_scale, v_scale, stream);
}

static gqap_status chunk_common(const gqap_chunk_plan_t* plan, const void* q, const void* k_pool,
                                const void* v_pool, const void* kr_pool, const int32_t* block_table,
                                const int32_t* cu_seqlens_q, const int32_t* kv_lens, float scale, bool fp8,
                                float k_scale, float v_scale, void* out, float* lse, void* workspace,
                                uint64_t workspace_bytes, void* stream) {
  if (!plan || plan->magic != GQAP_PLAN_MAGIC) return fail(GQAP_ERR_INVALID_ARGUMENT, "invalid chunk plan");
  const gqap_chunk_desc_t& d = plan->desc;
  if (chunk_fp8_cache(d) != fp8)
    return fail(GQAP_ERR_DTYPE, fp8 ? "gqap_chunk_prefill_fp8kv needs a plan with kv_dtype GQAP_FP8_E4M3FN"
                                    : "this plan has an fp8 cache: use gqap_chunk_prefill_fp8kv");
  if (!std::isfinite(scale)) return fail(GQAP_ERR_INVALID_ARGUMENT, "scale must be finite");
  if (fp8 && !(std::isfinite(k_scale) && k_scale > 0.f && std::isfinite(v_scale) && v_scale > 0.f))
    return fail(GQAP_ERR_INVALID_ARGUMENT, "k_scale and v_scale must be finite and > 0");
  if (d.batch == 0 || plan->q_tiles == 0) return GQAP_OK;
  if (!q || !k_pool || !v_pool || !block_table || !cu_seqlens_q || !kv_lens || !out)
    return fail(GQAP_ERR_INVALID_ARGUMENT, "null device pointer");
  if (d.head_dim_rope && !kr_pool) return fail(GQAP_ERR_INVALID_ARGUMENT, "kr_pool is required when head_dim_rope > 0");
  if (!d.head_dim_rope && kr_pool) return fail(GQAP_ERR_INVALID_ARGUMENT, "kr_pool given but head_dim_rope == 0");
  if (misaligned16(q) || misaligned16(k_pool) || misaligned16(v_pool) || misaligned16(out) ||
      (kr_pool && misaligned16(kr_pool)) ||
      ((uintptr_t)block_table & 3) || ((uintptr_t)cu_seqlens_q & 3) || ((uintptr_t)kv_lens & 3) ||
      (lse && ((uintptr_t)lse & 3)))
    return fail(GQAP_ERR_INVALID_ARGUMENT, "device pointers must be 16-byte aligned (index arrays, lse 4-byte)");
  if (plan->kernel == kChunkDecode || plan->kernel == kChunkDecodeFp8)
    return chunk_decode_launch(plan, q, k_pool, v_pool, kr_pool, block_table, cu_seqlens_q, kv_lens, scale, fp8,
                               k_scale, v_scale, out, lse, workspace, workspace_bytes, stream);
  PrefillArgs a{};
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k_pool;
  a.v = (const uint16_t*)v_pool;
  a.kr = (const uint16_t*)kr_pool;
  a.cu = cu_seqlens_q;
  a.mask = nullptr;
  a.out = (uint16_t*)out;
  a.lse = lse;
  a.q_st = d.q_stride_token;
  a.q_sh = d.q_stride_head;
  a.k_st = d.head_dim;  // rows of a page slab are contiguous
  a.k_sh = 0;
  a.v_st = d.head_dim;
  a.v_sh = 0;
  a.kr_st = d.head_dim_rope;  // rows of a rope page slab are contiguous
  a.kr_sb = d.kr_stride_block;
  a.o_st = d.out_stride_token;
  a.o_sh = d.out_stride_head;
  a.B = d.batch;
  a.Hq = d.num_q_heads;
  a.Hk = d.num_kv_heads;
  a.ratio = plan->ratio;
  a.q_tiles = plan->q_tiles;
  a.hpw = 128 / plan->q_tile_rows;
  a.mask_nb = 0;
  a.max_len = d.max_q_len;
  // fp8 cache: the key scale joins the softmax constant when the score is the
  // nope sum alone; with a rope part it multiplies the nope sum only.  The
  // value scale multiplies the normalised output.
  a.scale_log2 = scale * (fp8 && !d.head_dim_rope ? k_scale : 1.f) * dev::kLog2e;
  a.qk = fp8 ? k_scale : 1.f;
  a.v_scale = fp8 ? v_scale : 1.f;
  a.kvlens = kv_lens;
  a.bt = block_table;
  a.bt_st = d.block_table_stride;
  a.kv_sb = d.kv_stride_block;
  a.kv_sh = d.kv_stride_head;
  a.max_kv = d.max_kv_len;
  const gqap_status ss = split_setup((int32_t)plan->num_splits, d.total_q_tokens, d.num_q_heads,
                                     plan->workspace_bytes, workspace, workspace_bytes, &a);
  if (ss != GQAP_OK) return ss;
  const dim3 grid = prefill_grid(d.batch, d.num_q_heads, a.hpw, plan->q_tiles, a.nsplit, d.total_q_tokens);
  // Ranking by key count pays when workgroups start in rounds (more than
  // two per compute unit): it costs a short search per workgroup.
  a.rank_keys = (int64_t)grid.x > 2 * kDefaultCUs;
  hipStream_t st = (hipStream_t)stream;
  if (d.head_dim_rope == 64) {
    if (fp8)
      hipLaunchKernelGGL((prefill_fwd<64, true, 3>), grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((prefill_fwd<64, true, 0>), grid, dim3(256), 0, st, a);
  } else {
    if (fp8)
      hipLaunchKernelGGL((prefill_fwd<0, true, 3>), grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((prefill_fwd<0, true, 0>), grid, dim3(256), 0, st, a);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(GQAP_ERR_HIP, "chunk prefill launch: %s", hipGetErrorString(e));
  return launch_merge(a, d.max_q_len, st);
}

extern "C" gqap_status gqap_chunk_prefill(const gqap_chunk_plan_t* plan, const void* q, const void* k_pool,
                                          const void* v_pool, const void* kr_pool, const int32_t* block_table,
                                          const int32_t* cu_seqlens_q, const int32_t* kv_lens, float scale,
                                          void* out, float* lse, void* workspace, uint64_t workspace_bytes,
                                          void* stream) {
  return chunk_common(plan, q, k_pool, v_pool, kr_pool, block_table, cu_seqlens_q, kv_lens, scale, false, 1.f, 1.f,
                      out, lse, workspace, workspace_bytes, stream);
}

extern "C" gqap_status gqap_chunk_prefill_fp8kv(const gqap_chunk_plan_t* plan, const void* q, const void* k_pool,
                                                const void* v_pool, const void* kr_pool, const int32_t* block_table,
                                                const int32_t* cu_seqlens_q, const int32_t* kv_lens, float scale,
                                                float k_scale, float v_scale, void* out, float* lse, void* workspace,
                                                uint64_t workspace_bytes, void* stream) {
  return chunk_common(plan, q, k_pool, v_pool, kr_pool, block_table, cu_seqlens_q, kv_lens, scale, true, k_scale,
                      v_scale, out, lse, workspace, workspace_bytes, stream);
}
