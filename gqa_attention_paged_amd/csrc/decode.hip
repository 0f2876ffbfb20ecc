// Paged GQA decode for gfx950: balanced persistent workers + LSE combine.
//
// What is computed (FlashMLA tensor-shape reference, section 1 and the GQA
// diagram): for every sequence b and query head h, attention of the single
// query q[b, h] over the seq_lens[b] keys and values of KV head h / (Hq/Hk),
// gathered block by block through block_table.
//
// How (two launches on one stream):
//  1. decode_worker_*: one wave per worker.  A work unit is one 64-row key
//     block of one (sequence, KV head, head chunk); units are ordered
//     sequence-major, then (KV head, head chunk), then block.  The unit list
//     is cut into num_workers equal contiguous ranges, so every worker
//     streams the same number of K/V bytes whatever the lengths.  Each
//     worker finds its first unit with a wave-wide scan of seq_lens (no
//     separate metadata pass).  Each contiguous run of units of one
//     (sequence, KV head, head chunk) inside a worker's range is a piece; a
//     piece ends with a normalised partial output and its base-2 LSE in the
//     workspace, at slot (piece index + worker index), which is unique
//     because worker ranges are ordered.
//  2. decode_combine: merges the pieces of each (sequence, query head) with
//     weights 2^(lse_piece - max) and writes out (and the natural-log LSE).
//
// The bf16/fp8 worker keeps the next block in flight while it computes the
// current one: K goes straight into (double-buffered) registers in the
// 16x16x32 MFMA operand layout; V goes into staging registers as contiguous
// 16-byte rows, is written to an XOR-swizzled LDS tile once the current
// block's reads of that tile are issued, and comes back through the LDS
// transpose read as the token-packed operand of P.V.  All loads are plain
// register loads, so the compiler's wait counts stay exact.  The K/V reads
// carry the nontemporal hint: every cache byte is read once per pass, and
// the hinted stream keeps the eight XCDs within a few percent of each other
// (unhinted, their end times spread by about 10 %).  S^T = K q^T and
// O^T += V^T P^T run on bf16 MFMA with fp32 accumulation; the up-to-16 query
// heads of a KV head share every K/V byte.
//
// Chunk mode (the same kernels, template flag C): a short chunk of new tokens
// per sequence at the end of its keys (multi-token decode; FlashMLA
// tensor-shape reference, section 1, with a query length above 1).  A unit's
// 16 MFMA columns are then (token, query head) pairs of the KV head, each
// column with its own causal key limit, and the combine writes the chunk's
// rows.  The chunked-prefill plan picks this mode when the pairs fit the
// tiles one token's heads need.
#include "dev.hpp"
#include "status.hpp"

#include <cmath>
#include <mutex>
#include <type_traits>

namespace gqap {

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* block_table;
  const int32_t* seq_lens;
  int32_t* prefix;  // [B + 1] key blocks before each sequence (written by worker 0)
  float* ws_lse;    // [pieces][pcols] base 2
  float* ws_o;      // [pieces][pcols][D]
  void* out;
  float* lse;
  int64_t q_sb, q_sh, o_sb, o_sh;
  int64_t kv_block_bytes, kv_head_bytes, bt_stride;
  int32_t B, Hq, Hk, ratio, head_chunks, hkhc, nworkers;
  int32_t pcols;  // columns per piece slot in ws_lse / ws_o
  int32_t max_len;  // capacity from the plan; a longer (or negative) seq_len empties the sequence
  // Chunk mode (cu != null): sequence b holds the query rows cu[b] .. cu[b+1]-1
  // of a chunk aligned to the end of its seq_lens[b] keys; the first max_q of
  // them are computed.  A unit's 16 columns are then (token, head) pairs.
  const int32_t* cu;
  int32_t max_q;
  float score_scale_log2;  // scale * k_scale * log2(e) (with a rope part: scale * log2(e))
  float score_scale;       // scale * k_scale (with a rope part: scale)
  float v_scale;
  // MLA split head (rope kernels): the 64-wide rope row of every key, one
  // head shared by all query heads, in a paged rope cache of 64-row blocks;
  // an fp8 cache's k_scale then multiplies the per-head (nope) sum only.
  const void* kr;
  int64_t kr_block_bytes;
  float nope_scale;
};

namespace dev {

// Metadata that no decode kernel writes (seq_lens, block_table) is read
// through the constant address space: uniform reads become scalar loads,
// which wait on their own counter and never drain in-flight K/V loads.
__device__ __forceinline__ int ld_const(const int32_t* p, int64_t i) {
  return ((const int32_t __attribute__((address_space(4)))*)p)[i];
}

// Keys that the computed queries of sequence b read.  Decode: seq_lens[b].
// A length outside [0, max_len] (the capacity the plan was made for) is not
// truncated: the sequence is treated as empty, so its rows come out as 0 with
// lse = -inf, the same whatever the length was.  Chunk mode (C): a chunk of
// Lq rows ends at key seq_lens[b] - 1, and its row i sees the keys up to
// seq_lens[b] - Lq + i; with only the first min(Lq, max_q) rows computed, the
// keys read end at seq_lens[b] - Lq + min(Lq, max_q).  An empty chunk, or one
// with more rows than keys or more keys than the capacity, reads nothing.
template <bool C>
__device__ __forceinline__ int seq_keys(const DecodeArgs& a, int b) {
  const int L = ld_const(a.seq_lens, b);
  if constexpr (!C) {
    return (L < 0 || L > a.max_len) ? 0 : L;
  } else {
    const int Lq = ld_const(a.cu, b + 1) - ld_const(a.cu, b);
    if (Lq <= 0 || L > a.max_len || L < Lq) return 0;
    return L - Lq + min(Lq, a.max_q);
  }
}

// Position of one work unit.
struct Unit {
  int b;     // sequence
  int ql;    // kv_head * head_chunks + head_chunk
  int j;     // key block within the sequence
  int nblk;  // key blocks of sequence b
  int L;     // keys read for sequence b
  int phys;  // pool block holding block j
  int q0;    // first query row of sequence b (chunk mode)
  int qc;    // computed query rows of sequence b (chunk mode)
};

template <bool C>
__device__ __forceinline__ int seq_blocks(const DecodeArgs& a, int b) { return (seq_keys<C>(a, b) + 63) >> 6; }

template <bool C>
__device__ __forceinline__ void unit_load_seq(const DecodeArgs& a, Unit& u) {
  u.L = seq_keys<C>(a, u.b);
  u.nblk = (u.L + 63) >> 6;
  if constexpr (C) {
    u.q0 = ld_const(a.cu, u.b);
    u.qc = min(ld_const(a.cu, u.b + 1) - u.q0, a.max_q);
  }
}

__device__ __forceinline__ void unit_load_phys(const DecodeArgs& a, Unit& u) {
  u.phys = ld_const(a.block_table, (int64_t)u.b * a.bt_stride + u.j);
}

// A value that every lane of the wave holds alike, moved to a scalar
// register.  What is computed from it then stays scalar, so the unit
// bookkeeping reads seq_lens and block_table with scalar loads (which wait
// on their own counter) instead of vector loads queued behind the K/V stream.
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ int64_t uniform(int64_t x) {
  const uint64_t u = (uint64_t)x;
  return (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(u >> 32)) << 32) |
                   (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)u));
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int x) {
  const int lane = __lane_id();
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  return x;
}

// Key blocks of sequences [0, b_end), summed by one wave (all lanes get it).
template <bool C>
__device__ __forceinline__ int64_t blocks_before(const DecodeArgs& a, int b_end) {
  int64_t total = 0;
  const int lane = __lane_id();
  for (int b0 = 0; b0 < b_end; b0 += 64) {
    const int b = b0 + lane;
    int nb = b < b_end ? seq_blocks<C>(a, b) : 0;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) nb += __shfl_xor(nb, off);
    total += uniform(nb);
  }
  return total;
}

// Sequence holding key-block ordinal t (prefix[b] <= t < prefix[b+1]) and
// prefix[b], found by one wave scanning seq_lens 64 sequences at a time.
template <bool C>
__device__ __forceinline__ void locate_block(const DecodeArgs& a, int64_t t, int* b_out, int64_t* before_out) {
  int64_t run = 0;
  const int lane = __lane_id();
  for (int b0 = 0; b0 < a.B; b0 += 64) {
    const int b = b0 + lane;
    const int nb = b < a.B ? seq_blocks<C>(a, b) : 0;
    const int incl = wave_incl_scan(nb);
    const bool hit = nb > 0 && run + incl - nb <= t && t < run + incl;
    const unsigned long long m = __ballot(hit);
    if (m) {
      const int l = __ffsll((long long)m) - 1;
      *b_out = b0 + l;
      *before_out = run + uniform(__shfl(incl - nb, l));
      return;
    }
    run += uniform(__shfl(incl, 63));
  }
  *b_out = a.B;
  *before_out = run;
}

// Exclusive prefix of the per-sequence block counts -> a.prefix[0..B] (one wave).
template <bool C>
__device__ __forceinline__ void write_prefix(const DecodeArgs& a) {
  int64_t run = 0;
  const int lane = __lane_id();
  for (int b0 = 0; b0 < a.B; b0 += 64) {
    const int b = b0 + lane;
    const int nb = b < a.B ? seq_blocks<C>(a, b) : 0;
    const int incl = wave_incl_scan(nb);
    if (b < a.B) a.prefix[b] = (int32_t)(run + incl - nb);
    run += __shfl(incl, 63);
  }
  if (lane == 0) a.prefix[a.B] = (int32_t)run;
}

// First unit of a worker whose range starts at unit ub.
template <bool C>
__device__ __forceinline__ Unit unit_at(const DecodeArgs& a, int64_t ub) {
  Unit u;
  int64_t before;
  locate_block<C>(a, ub / a.hkhc, &u.b, &before);
  unit_load_seq<C>(a, u);
  const int rem = (int)(ub - before * a.hkhc);
  u.ql = rem / u.nblk;
  u.j = rem - u.ql * u.nblk;
  unit_load_phys(a, u);
  return u;
}

// Next unit in sequence-major order, skipping sequences without keys.  Only
// called while the worker's range still holds a unit, so b stays below B.
template <bool C>
__device__ __forceinline__ Unit unit_next(const DecodeArgs& a, Unit u) {
  if (++u.j == u.nblk) {
    u.j = 0;
    if (++u.ql == a.hkhc) {
      u.ql = 0;
      do {
        ++u.b;
      } while (u.b < a.B && seq_blocks<C>(a, u.b) == 0);
      if (u.b < a.B) unit_load_seq<C>(a, u);
    }
  }
  if (u.b < a.B) unit_load_phys(a, u);
  return u;
}

__device__ __forceinline__ bool same_piece(const Unit& x, const Unit& y) { return x.b == y.b && x.ql == y.ql; }

// Token (row of the 64-row block) held by MFMA row m of score tile mt.  The
// PV operand needs each 16-lane group to hold 8 tokens that the V transpose
// read delivers: two runs of 4 for 16-bit V, one run of 8 for 8-bit V.
template <bool FP8>
__device__ __forceinline__ int token_of(int mt, int m) {
  if (FP8) return 32 * (mt >> 1) + 8 * (m >> 2) + 4 * (mt & 1) + (m & 3);
  return 16 * mt + m;
}

// Byte offset of (row, byte column c) inside a V tile in LDS.  Rows are RB
// bytes; pieces of P bytes are XOR-permuted within their row so that the
// transpose reads (16 or 32 rows at one column) spread over all banks.
template <int RB, int P>
__device__ __forceinline__ int vswz(int row, int c) {
  constexpr int NP = RB / P;
  constexpr int RW = 256 / RB;
  const int piece = (c / P) ^ ((row / RW) % NP);
  return row * RB + piece * P + (c % P);
}

}  // namespace dev

using namespace dev;

// C: chunk mode.  Column col of head chunk hc is then the pair (token i,
// head hh) with hc * 16 + col = i * ratio + hh, and its keys end at its own
// causal bound, so every column carries its own key limit.  DR: width of the
// MLA rope part (0 or 64), scored after the per-head part on its own rows.
template <int D, bool FP8, bool C, int DR>
__device__ __forceinline__ void decode_worker_body(const DecodeArgs& a) {
  constexpr int ESZ = FP8 ? 1 : 2;
  constexpr int RB = D * ESZ;        // bytes per K/V row
  constexpr int HB = 32 * RB;        // bytes per half slab (32 rows)
  constexpr int PB = FP8 ? 16 : 32;  // swizzle piece
  constexpr int KSTEPS = D / 32;     // MFMA k-steps over the head dim
  constexpr int KLOADS = RB / 64;    // 16-byte K loads per row and lane group
  constexpr int NT = D / 16;         // 16-wide output tiles
  constexpr int NV = HB / 1024;      // 16-byte V loads per lane and half slab
  constexpr int KSR = DR / 32;       // MFMA k-steps over the rope part (bf16)
  __shared__ __attribute__((aligned(1024))) unsigned char vlds[HB];

  const int w = blockIdx.x;
  const int lane = threadIdx.x;
  const int col = lane & 15;
  const int G = lane >> 4;
  if (w == 0) write_prefix<C>(a);  // for the combine pass
  const int64_t W = blocks_before<C>(a, a.B) * a.hkhc;
  const int64_t ub = W * w / a.nworkers;
  const int64_t ue = W * (w + 1) / a.nworkers;
  if (ub >= ue) return;
  const int count = (int)(ue - ub);

  const unsigned char* kpool = (const unsigned char*)a.k;
  const unsigned char* vpool = (const unsigned char*)a.v;

  i32x4 kreg[2][KLOADS];  // K rows of the half about to be scored (two 16-row tiles)
  i32x4 vst[NV];          // V rows of the next half, on their way to LDS
  i32x4 kregr[2][KSR > 0 ? KSR : 1];  // rope rows of the same half
  bf16x8 qop[KSTEPS + KSR];
  float m_run, l_run;
  f32x4 o[NT];
  f32x4 s[2];
  int klim = 0;  // chunk mode: keys of this lane's column, [0, klim) of the sequence

  auto reset = [&]() {
    m_run = -INFINITY;
    l_run = 0.f;
#pragma unroll
    for (int n = 0; n < NT; ++n) o[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  };

  auto slab_offset = [&](const Unit& u) {
    const int g = u.ql / a.head_chunks;
    return (int64_t)u.phys * a.kv_block_bytes + (int64_t)g * a.kv_head_bytes;
  };

  // (token, head) of this lane's column in the piece's head chunk; decode
  // has one token, so the column is the head.
  auto column = [&](const Unit& u, int* tok, int* hl) {
    const int g = u.ql / a.head_chunks;
    const int gc = (u.ql - g * a.head_chunks) * 16 + col;
    *tok = C ? gc / a.ratio : 0;
    *hl = gc - *tok * a.ratio;
    return C ? *tok < u.qc : gc < a.ratio;
  };

  // Chunk mode: row i of the chunk sees keys [0, L - qc + 1 + i); a column
  // without a query keeps the sequence's whole range (its q is zero).
  auto set_limit = [&](const Unit& u) {
    if constexpr (C) {
      int tok, hl;
      klim = column(u, &tok, &hl) ? u.L - u.qc + 1 + tok : u.L;
    }
  };

  // Query heads of the piece's chunk as the B operand (k slots match the K loads).
  auto load_q = [&](const Unit& u) {
    const int g = u.ql / a.head_chunks;
    int tok, hl;
    const bool hvalid = column(u, &tok, &hl);
    const int64_t row = C ? (int64_t)u.q0 + (hvalid ? tok : 0) : (int64_t)u.b;
    const unsigned char* qp = (const unsigned char*)a.q +
                              (row * a.q_sb + (int64_t)(g * a.ratio + (hvalid ? hl : 0)) * a.q_sh) * 2;
#pragma unroll
    for (int ks = 0; ks < KSTEPS + KSR; ++ks) {
      // rope steps (ks >= KSTEPS): the bf16 layout, after the D per-head values
      const int d0 = ks >= KSTEPS ? D + 32 * (ks - KSTEPS) + 8 * G
                     : FP8        ? (64 * (ks >> 1) + 16 * G + 8 * (ks & 1))
                                  : (32 * ks + 8 * G);
      const i32x4 v = hvalid ? load16(qp + 2 * d0) : i32x4{0, 0, 0, 0};
      qop[ks] = __builtin_bit_cast(bf16x8, v);
    }
  };

  // K rows of half h of a unit, straight into the MFMA A-operand layout.
  auto issue_k = [&](const Unit& u, auto hc_) {
    constexpr int H = decltype(hc_)::value;
    const unsigned char* kblk = kpool + slab_offset(u);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const unsigned char* kp = kblk + token_of<FP8>(2 * H + t, col) * RB + 16 * G;
#pragma unroll
      for (int p = 0; p < KLOADS; ++p) kreg[t][p] = load16_stream(kp + 64 * p);
    }
    // The rope rows of the same tokens.  Every query head of the sequence
    // reads them, so they are read without the streaming hint and may be
    // served from the caches.
    if constexpr (DR > 0) {
      const unsigned char* rblk = (const unsigned char*)a.kr + (int64_t)u.phys * a.kr_block_bytes;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const unsigned char* rp = rblk + token_of<FP8>(2 * H + t, col) * (2 * DR) + 16 * G;
#pragma unroll
        for (int r = 0; r < KSR; ++r) kregr[t][r] = load16(rp + 64 * r);
      }
    }
  };

  // V rows of half h of a unit as contiguous 16-byte chunks into the staging registers.
  auto issue_v = [&](const Unit& u, auto hc_) {
    constexpr int H = decltype(hc_)::value;
    const unsigned char* vh = vpool + slab_offset(u) + H * HB;
#pragma unroll
    for (int i = 0; i < NV; ++i) vst[i] = load16_stream(vh + 1024 * i + 16 * lane);
  };

  // Staged V rows -> the swizzled LDS tile (rows 0..31 of the half).
  auto stage_v = [&]() {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int byte = 1024 * i + 16 * lane;
      store16(vlds + vswz<RB, PB>(byte / RB, byte % RB), vst[i]);
    }
  };

  // S^T[token, head] = K q^T for the 32 rows whose K is in kreg.
  auto qk = [&]() {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      s[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        bf16x8 ka;
        if constexpr (FP8) {
          const i32x4 wv = kreg[t][ks >> 1];
          ka = fp8x8_to_bf16x8(i32x2{wv[2 * (ks & 1)], wv[2 * (ks & 1) + 1]});
        } else {
          ka = __builtin_bit_cast(bf16x8, kreg[t][ks]);
        }
        s[t] = mfma16x16x32(ka, qop[ks], s[t]);
      }
      if constexpr (DR > 0) {
        if constexpr (FP8) s[t] *= a.nope_scale;  // k_scale belongs to the per-head sum only
#pragma unroll
        for (int r = 0; r < KSR; ++r)
          s[t] = mfma16x16x32(__builtin_bit_cast(bf16x8, kregr[t][r]), qop[KSTEPS + r], s[t]);
      }
    }
  };

  // Online softmax (base 2) of one half's scores and O^T += V^T P^T from LDS.
  auto softmax_pv = [&](const Unit& u, auto hc_) {
    constexpr int H = decltype(hc_)::value;
    const int valid = min(64, u.L - 64 * u.j) - 32 * H;  // may be <= 0: then the half is all padding
    // Keys past seq_len (chunk mode: past the column's own limit) are dropped
    // by select: whatever the padding rows hold never reaches the sums.
    const int kvalid = C ? min(64, klim - 64 * u.j) - 32 * H : valid;
    float bmax = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float x = token_of<FP8>(t, 4 * G + j) < kvalid ? s[t][j] * a.score_scale_log2 : -INFINITY;
        s[t][j] = x;
        bmax = fmaxf(bmax, x);
      }
    bmax = wave_max4(bmax);
    const float m_new = fmaxf(m_run, bmax);
    // Chunk mode: a column may have seen no key yet (its keys end before this
    // piece's); subtracting 0 instead of -inf keeps its sums at exactly 0.
    const float m_sub = C && m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_sub);
    float psum = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p = fast_exp2(s[t][j] - m_sub);
        s[t][j] = p;
        psum += p;
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int n = 0; n < NT; ++n) o[n] *= alpha;

    // P^T as the B operand: k-slot e of lane group G is token_of(e/4, 4G + e%4).
    i32x4 pw;
    pw[0] = (int)pack_bf16x2_hw(s[0][0], s[0][1]);
    pw[1] = (int)pack_bf16x2_hw(s[0][2], s[0][3]);
    pw[2] = (int)pack_bf16x2_hw(s[1][0], s[1][1]);
    pw[3] = (int)pack_bf16x2_hw(s[1][2], s[1][3]);
    const bf16x8 pop = __builtin_bit_cast(bf16x8, pw);

    // O^T[d, head] += V^T P^T; V rows past seq_len are zeroed after the read.
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      bf16x8 va;
      if constexpr (FP8) {
        const int t0 = 8 * G;
        i32x2 wv = lds_read_tr8(vlds + vswz<RB, PB>(t0 + (col >> 1), 16 * n + 8 * (col & 1)));
        if (valid < 32) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (t0 + e >= valid) wv[e >> 2] &= ~(0xff << (8 * (e & 3)));
        }
        va = fp8x8_to_bf16x8(wv);
      } else {
        i32x4 wv;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int t0 = 16 * hf + 4 * G;
          const i16x4 r = lds_read_tr16(vlds + vswz<RB, PB>(t0 + (col >> 2), 32 * n + 8 * (col & 3)));
          uint32_t lo = (uint16_t)r[0] | ((uint32_t)(uint16_t)r[1] << 16);
          uint32_t hi = (uint16_t)r[2] | ((uint32_t)(uint16_t)r[3] << 16);
          if (valid < 32) {
            if (t0 + 0 >= valid) lo &= 0xffff0000u;
            if (t0 + 1 >= valid) lo &= 0x0000ffffu;
            if (t0 + 2 >= valid) hi &= 0xffff0000u;
            if (t0 + 3 >= valid) hi &= 0x0000ffffu;
          }
          wv[2 * hf] = (int)lo;
          wv[2 * hf + 1] = (int)hi;
        }
        va = __builtin_bit_cast(bf16x8, wv);
      }
      o[n] = mfma16x16x32(va, pop, o[n]);
    }
  };

  // Normalised partial of the finished piece -> its workspace slot.
  auto flush = [&](const Unit& u) {
    const float l_tot = wave_sum4(l_run);
    int tok, hl;
    const bool cvalid = column(u, &tok, &hl);
    const int64_t slot = (int64_t)u.b * a.hkhc + u.ql + w;
    if (cvalid) {
      // A chunk column with no key in this piece leaves 0 and lse -inf.
      const float inv = C && l_tot == 0.f ? 0.f : a.v_scale / l_tot;
      float* dst = a.ws_o + (slot * a.pcols + col) * D + 4 * G;
#pragma unroll
      for (int n = 0; n < NT; ++n) *(f32x4*)(dst + 16 * n) = o[n] * inv;
      if (G == 0) a.ws_lse[slot * a.pcols + col] = m_run + log2f(l_tot);
    }
  };

  using H0 = std::integral_constant<int, 0>;
  using H1 = std::integral_constant<int, 1>;

  // Pipeline over 32-row halves (half X = current, X+1, X+2 the next two):
  // K(X+1) is issued as soon as the scores of X have consumed the K
  // registers, and V(X+2) as soon as V(X+1) has left the staging registers
  // for the LDS tile (after X's reads of it), so roughly one half of K and V
  // is always in flight per wave.  The steady-state loop issues
  // unconditionally (every path into a wait has the same loads outstanding,
  // which keeps the compiler's wait counts exact); the last unit is peeled.
  // A new query operand is loaded right after the scores that last used the
  // old one, ahead of that step's K issue.
  Unit cur = unit_at<C>(a, ub);
  reset();
  set_limit(cur);
  load_q(cur);
  issue_k(cur, H0{});
  issue_v(cur, H0{});
  Unit nx = count > 1 ? unit_next<C>(a, cur) : cur;
  stage_v();
  issue_v(cur, H1{});
  int i = 0;
  for (; i + 1 < count; ++i) {
    const bool boundary = !same_piece(cur, nx);
    // first half of cur
    qk();
    issue_k(cur, H1{});
    softmax_pv(cur, H0{});
    stage_v();
    issue_v(nx, H0{});
    // second half of cur
    qk();
    if (boundary) load_q(nx);
    issue_k(nx, H0{});
    softmax_pv(cur, H1{});
    stage_v();
    issue_v(nx, H1{});
    if (boundary) {
      flush(cur);
      reset();
      set_limit(nx);
    }
    const Unit nx2 = (i + 2 < count) ? unit_next<C>(a, nx) : nx;
    cur = nx;
    nx = nx2;
  }
  qk();
  issue_k(cur, H1{});
  softmax_pv(cur, H0{});
  stage_v();
  qk();
  softmax_pv(cur, H1{});
  flush(cur);
}

template <int D, bool FP8, bool C>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void decode_worker_mfma(DecodeArgs a) {
  decode_worker_body<D, FP8, C, 0>(a);
}

// Short chunks with the MLA split head: 128 per-head dims plus the 64-wide
// rope row of every key from the paged rope cache.  The plan runs at most
// one worker per SIMD, so the kernel may take a SIMD's whole register file.
template <bool FP8>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(1))) void decode_worker_rope(DecodeArgs a) {
  decode_worker_body<128, FP8, true, 64>(a);
}

// fp32 path: one wave per worker, vector ALU, no prefetch.  Lane t scores
// token t of a block (K staged in LDS); lane d accumulates output columns
// d, d+64 reading V rows straight from the pool (rows past seq_len are never
// touched).
template <int D>
__global__ __launch_bounds__(64) void decode_worker_f32(DecodeArgs a) {
  constexpr int DC = D / 64;
  __shared__ float sK[64][D + 1];
  __shared__ float sQ[16][D];
  __shared__ float sP[16][64];

  const int w = blockIdx.x;
  const int lane = threadIdx.x;
  if (w == 0) write_prefix<false>(a);  // for the combine pass
  const int64_t W = blocks_before<false>(a, a.B) * a.hkhc;
  const int64_t ub = W * w / a.nworkers;
  const int64_t ue = W * (w + 1) / a.nworkers;
  if (ub >= ue) return;
  const int count = (int)(ue - ub);
  const unsigned char* kpool = (const unsigned char*)a.k;
  const unsigned char* vpool = (const unsigned char*)a.v;
  const float* q = (const float*)a.q;

  float m[16], l[16], o[16][DC];
  auto reset = [&]() {
#pragma unroll
    for (int hh = 0; hh < 16; ++hh) {
      m[hh] = -INFINITY;
      l[hh] = 0.f;
#pragma unroll
      for (int c = 0; c < DC; ++c) o[hh][c] = 0.f;
    }
  };
  auto load_q = [&](const Unit& u) {
    const int g = u.ql / a.head_chunks;
    const int hc = u.ql - g * a.head_chunks;
    const int rc = min(16, a.ratio - hc * 16);
    const int hbase = g * a.ratio + hc * 16;
    __syncthreads();
    for (int i = lane; i < 16 * D; i += 64) {
      const int hh = i / D, d = i % D;
      sQ[hh][d] = hh < rc ? q[(int64_t)u.b * a.q_sb + (int64_t)(hbase + hh) * a.q_sh + d] : 0.f;
    }
    __syncthreads();
  };
  auto flush = [&](const Unit& u) {
    const int g = u.ql / a.head_chunks;
    const int hc = u.ql - g * a.head_chunks;
    const int rc = min(16, a.ratio - hc * 16);
    const int64_t slot = (int64_t)u.b * a.hkhc + u.ql + w;
#pragma unroll
    for (int hh = 0; hh < 16; ++hh) {
      if (hh >= rc) break;
#pragma unroll
      for (int c = 0; c < DC; ++c)
        a.ws_o[(slot * a.pcols + hh) * D + lane + 64 * c] = o[hh][c] / l[hh] * a.v_scale;
      if (lane == 0) a.ws_lse[slot * a.pcols + hh] = m[hh] * kLog2e + log2f(l[hh]);
    }
  };

  Unit u = unit_at<false>(a, ub);
  reset();
  load_q(u);
  for (int i = 0; i < count; ++i) {
    const int g = u.ql / a.head_chunks;
    const int hc = u.ql - g * a.head_chunks;
    const int rc = min(16, a.ratio - hc * 16);
    const int64_t off = (int64_t)u.phys * a.kv_block_bytes + (int64_t)g * a.kv_head_bytes;
    const float* kblk = (const float*)(kpool + off);
    const float* vblk = (const float*)(vpool + off);
    const int valid = min(64, u.L - 64 * u.j);
    __syncthreads();
    for (int i2 = lane; i2 < 64 * D; i2 += 64) {
      const int t = i2 / D, d = i2 % D;
      sK[t][d] = t < valid ? kblk[i2] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int hh = 0; hh < 16; ++hh) {
      if (hh >= rc) break;
      float acc = 0.f;
      for (int d = 0; d < D; ++d) acc = fmaf(sQ[hh][d], sK[lane][d], acc);
      const float sc = lane < valid ? acc * a.score_scale : -INFINITY;
      float bmax = sc;
#pragma unroll
      for (int off2 = 32; off2 > 0; off2 >>= 1) bmax = fmaxf(bmax, __shfl_xor(bmax, off2));
      const float m_new = fmaxf(m[hh], bmax);
      const float alpha = expf(m[hh] - m_new);
      const float p = lane < valid ? expf(sc - m_new) : 0.f;
      float ps = p;
#pragma unroll
      for (int off2 = 32; off2 > 0; off2 >>= 1) ps += __shfl_xor(ps, off2);
      l[hh] = l[hh] * alpha + ps;
      m[hh] = m_new;
      sP[hh][lane] = p;
#pragma unroll
      for (int c = 0; c < DC; ++c) o[hh][c] *= alpha;
    }
    __syncthreads();
#pragma unroll
    for (int hh = 0; hh < 16; ++hh) {
      if (hh >= rc) break;
      for (int t = 0; t < valid; ++t) {
        const float p = sP[hh][t];
#pragma unroll
        for (int c = 0; c < DC; ++c) o[hh][c] = fmaf(p, vblk[t * D + lane + 64 * c], o[hh][c]);
      }
    }
    if (i + 1 == count) {
      flush(u);
      break;
    }
    const Unit nx = unit_next<false>(a, u);
    if (!same_piece(u, nx)) {
      flush(u);
      reset();
      load_q(nx);
    }
    u = nx;
  }
}

// Merge the pieces of one (sequence, query head): weights 2^(lse - max).
// One wave; lane k holds the LSE of piece k (64 pieces per round), and the
// output rows of all pieces are requested before any arithmetic, so the
// merge costs one memory round trip for the usual handful of pieces.
// Chunk mode (C): workgroup (sequence, query head, y) takes row y of the
// sequence's chunk, and the last y also every row past max_q; rows past the
// computed ones (and every row of a chunk that reads no key) get 0 and lse
// -inf.
template <int D, bool OUT_BF16, bool C>
__global__ __launch_bounds__(64) void decode_combine(DecodeArgs a) {
  constexpr int DC = D / 64;
  const int bh = blockIdx.x;
  const int b = bh / a.Hq;
  const int h = bh - b * a.Hq;
  const int lane = threadIdx.x;
  const int g = h / a.ratio;
  const int hh = h - g * a.ratio;
  const int pb = ld_const(a.prefix, b);
  const int nblk = ld_const(a.prefix, b + 1) - pb;
  const int row0 = C ? ld_const(a.cu, b) : b;
  const int rows = C ? ld_const(a.cu, b + 1) - row0 : 1;
  const int qc = C ? min(rows, a.max_q) : 1;
  const int i0 = C ? (int)blockIdx.y : 0;
  const int i_end = !C ? 1 : (int)blockIdx.y + 1 == (int)gridDim.y ? rows : min(rows, i0 + 1);
  for (int i = i0; i < i_end; ++i) {
    const bool computed = nblk > 0 && i < qc;
    const int gc = computed ? i * a.ratio + hh : 0;  // column of (token i, head hh)
    const int hc = gc >> 4;
    const int col = gc & 15;
    const int ql = g * a.head_chunks + hc;
    const int64_t qg = (int64_t)b * a.hkhc + ql;
    float acc[DC];
#pragma unroll
    for (int c = 0; c < DC; ++c) acc[c] = 0.f;
    float M = -INFINITY, den = 0.f;
    if (computed) {
      const int64_t W = (int64_t)ld_const(a.prefix, a.B) * a.hkhc;
      const int64_t u0 = (int64_t)pb * a.hkhc + (int64_t)ql * nblk;
      const int64_t u1 = u0 + nblk;
      const int64_t P = a.nworkers;
      const int w0 = (int)(((u0 + 1) * P - 1) / W);  // worker holding unit u0
      const int w1 = (int)((u1 * P - 1) / W);        // worker holding unit u1 - 1
      // With fewer units than workers some workers own no unit; they wrote nothing.
      auto owns_units = [&](int wk) { return W * wk / P < W * (wk + 1) / P; };
      if (w1 - w0 < 4) {
        // Up to four pieces (the usual case): their LSEs and rows are requested
        // together, so the merge costs a single memory round trip.
        const int n = w1 - w0 + 1;
        const bool live = lane < n && owns_units(w0 + lane);
        const float lse_k = live ? a.ws_lse[(qg + w0 + lane) * a.pcols + col] : -INFINITY;
        float v4[4][DC];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const float* op = a.ws_o + ((qg + w0 + min(kk, n - 1)) * a.pcols + col) * D;
#pragma unroll
          for (int c = 0; c < DC; ++c) v4[kk][c] = op[lane + 64 * c];
        }
        M = lse_k;
#pragma unroll
        for (int off = 2; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
        M = __shfl(M, 0);
        const float wt_k = live ? exp2f(lse_k - M) : 0.f;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const float w = __shfl(wt_k, kk);  // 0 for kk >= n or a piece-less worker
          den += w;
#pragma unroll
          for (int c = 0; c < DC; ++c) acc[c] += w > 0.f ? w * v4[kk][c] : 0.f;
        }
      } else
      for (int r0 = w0; r0 <= w1; r0 += 64) {
        const int wk = r0 + lane;
        const bool live = wk <= w1 && owns_units(wk);
        const float lse_k = live ? a.ws_lse[(qg + wk) * a.pcols + col] : -INFINITY;
        float m_round = lse_k;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) m_round = fmaxf(m_round, __shfl_xor(m_round, off));
        const float M_new = fmaxf(M, m_round);
        const float scale_old = M == -INFINITY ? 0.f : exp2f(M - M_new);
#pragma unroll
        for (int c = 0; c < DC; ++c) acc[c] *= scale_old;
        den *= scale_old;
        const float wt_k = live ? exp2f(lse_k - M_new) : 0.f;
        float wsum = wt_k;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) wsum += __shfl_xor(wsum, off);
        den += wsum;
        const int n = min(64, w1 - r0 + 1);
        // Four pieces per trip, all loads first.  Slots of empty workers are
        // read (they are inside the workspace) but dropped by select, so stale
        // contents never reach the sum.
        for (int k0 = 0; k0 < n; k0 += 4) {
          float v4[4][DC], w4[4];
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) {
            const int k = min(k0 + kk, n - 1);
            w4[kk] = k0 + kk < n ? __shfl(wt_k, k) : 0.f;
            const float* op = a.ws_o + ((qg + r0 + k) * a.pcols + col) * D;
#pragma unroll
            for (int c = 0; c < DC; ++c) v4[kk][c] = op[lane + 64 * c];
          }
#pragma unroll
          for (int kk = 0; kk < 4; ++kk)
#pragma unroll
            for (int c = 0; c < DC; ++c) acc[c] += w4[kk] > 0.f ? w4[kk] * v4[kk][c] : 0.f;
        }
        M = M_new;
      }
    }
    // A chunk row can have a zero denominator only if all its pieces saw no
    // key, which the causal bound rules out; the guard keeps it at 0 anyway.
    const bool some = computed && den > 0.f;
    const int64_t row = (int64_t)row0 + i;
    const int64_t obase = row * a.o_sb + (int64_t)h * a.o_sh;
#pragma unroll
    for (int c = 0; c < DC; ++c) {
      const float v = some ? acc[c] / den : 0.f;
      if (OUT_BF16)
        ((uint16_t*)a.out)[obase + lane + 64 * c] = f32_to_bf16(v);
      else
        ((float*)a.out)[obase + lane + 64 * c] = v;
    }
    if (a.lse && lane == 0) a.lse[row * a.Hq + h] = some ? (M + log2f(den)) * kLn2 : -INFINITY;
  }
}

// Padded block table from the flat CSR page list (MATE msa_interface,
// _build_page_table_from_flat_kv_indices): row b holds the pages
// kv_indices[indptr[b] .. indptr[b+1]) in order, then -1.  One thread per
// table entry.
__global__ __launch_bounds__(256) void block_table_from_csr(const int32_t* kv_indices, const int32_t* indptr,
                                                           int32_t batch, int32_t width, int64_t stride,
                                                           int32_t* table) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)batch * width) return;
  const int b = (int)(i / width), j = (int)(i - (int64_t)b * width);
  const int p0 = indptr[b], n = indptr[b + 1] - p0;
  table[(int64_t)b * stride + j] = j < n ? kv_indices[(int64_t)p0 + j] : -1;
}

// Copy logical rows of one (sequence, KV head) out of the pool with the same
// slab address function the decode kernels use.
__global__ __launch_bounds__(256) void debug_gather_kv(const unsigned char* pool, const int32_t* block_table,
                                                      const int32_t* seq_lens, int64_t bt_stride,
                                                      int64_t block_bytes, int64_t head_bytes, int row_bytes, int b,
                                                      int g, int num_rows, unsigned char* dst) {
  const int chunks = row_bytes / 16;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int t = (int)(idx / chunks);
  const int c = (int)(idx % chunks);
  const int rows = min(num_rows, seq_lens[b]);
  if (t >= rows) return;
  const int32_t* bt = block_table + (int64_t)b * bt_stride;
  const unsigned char* src = kv_slab(pool, bt, t >> 6, g, block_bytes, head_bytes) + (t & 63) * row_bytes;
  store16(dst + (int64_t)t * row_bytes + 16 * c, load16(src + 16 * c));
}

static int dtype_size(int32_t dt) { return dt == GQAP_F32 ? 4 : dt == GQAP_BF16 ? 2 : 1; }

static bool misaligned(const void* p, uintptr_t a) { return ((uintptr_t)p) & (a - 1); }

// Workspace of the decode variant that allocates nothing: one array per GPU,
// held from the first call on that GPU until the process ends.  Host code
// never uses its name as an address (on the host it is a stand-in): the
// device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[GQAP_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

// Device address of `scratch` on the current device, looked up on the first
// call made with that device current and kept.
static gqap_status scratch_address(void** out) {
  static std::mutex mu;
  static void* ptr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(GQAP_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(GQAP_ERR_UNSUPPORTED, "device %d beyond the %d supported", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(mu);
  if (!ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(GQAP_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    ptr[dev] = p;
  }
  *out = ptr[dev];
  return GQAP_OK;
}

static gqap_status decode_launch(const gqap_decode_plan_t* plan, const void* q, const void* k_pool,
                                 const void* v_pool, const int32_t* block_table, const int32_t* seq_lens,
                                 float scale, float k_scale, float v_scale, void* out, float* lse, void* workspace,
                                 uint64_t workspace_bytes, void* stream);

}  // namespace gqap

using namespace gqap;

extern "C" gqap_status gqap_paged_decode(const gqap_decode_plan_t* plan, const void* q, const void* k_pool,
                                         const void* v_pool, const int32_t* block_table, const int32_t* seq_lens,
                                         float scale, float k_scale, float v_scale, void* out, float* lse,
                                         void* workspace, uint64_t workspace_bytes, void* stream) {
  return decode_launch(plan, q, k_pool, v_pool, block_table, seq_lens, scale, k_scale, v_scale, out, lse, workspace,
                       workspace_bytes, stream);
}

extern "C" gqap_status gqap_paged_decode_noalloc(const gqap_decode_plan_t* plan, const void* q, const void* k_pool,
                                                 const void* v_pool, const int32_t* block_table,
                                                 const int32_t* seq_lens, float scale, float k_scale, float v_scale,
                                                 void* out, float* lse, void* stream) {
  if (!plan || plan->magic != GQAP_PLAN_MAGIC) return fail(GQAP_ERR_INVALID_ARGUMENT, "invalid decode plan");
  if (plan->workspace_bytes > (uint64_t)GQAP_NOALLOC_SCRATCH_BYTES)
    return fail(GQAP_ERR_UNSUPPORTED,
                "this plan needs %llu bytes of workspace; the allocation-free decode has %llu "
                "(use gqap_paged_decode with a caller workspace, or fewer sequences, heads or workers)",
                (unsigned long long)plan->workspace_bytes, (unsigned long long)GQAP_NOALLOC_SCRATCH_BYTES);
  if (plan->desc.batch == 0) return GQAP_OK;
  void* ws = nullptr;
  const gqap_status s = scratch_address(&ws);
  if (s != GQAP_OK) return s;
  return decode_launch(plan, q, k_pool, v_pool, block_table, seq_lens, scale, k_scale, v_scale, out, lse, ws,
                       (uint64_t)GQAP_NOALLOC_SCRATCH_BYTES, stream);
}

gqap_status gqap::decode_launch(const gqap_decode_plan_t* plan, const void* q, const void* k_pool,
                                const void* v_pool, const int32_t* block_table, const int32_t* seq_lens,
                                float scale, float k_scale, float v_scale, void* out, float* lse,
                                void* workspace, uint64_t workspace_bytes, void* stream) {
  if (!plan || plan->magic != GQAP_PLAN_MAGIC) return fail(GQAP_ERR_INVALID_ARGUMENT, "invalid decode plan");
  const gqap_decode_desc_t& d = plan->desc;
  if (d.batch == 0) return GQAP_OK;
  if (!q || !k_pool || !v_pool || !block_table || !seq_lens || !out || !workspace)
    return fail(GQAP_ERR_INVALID_ARGUMENT, "null device pointer");
  if (misaligned(q, 16) || misaligned(k_pool, 16) || misaligned(v_pool, 16) || misaligned(out, 16) ||
      misaligned(block_table, 4) || misaligned(seq_lens, 4) || (lse && misaligned(lse, 4)))
    return fail(GQAP_ERR_INVALID_ARGUMENT, "device pointers must be 16-byte aligned (index vectors 4-byte)");
  if (misaligned(workspace, 256)) return fail(GQAP_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  if (workspace_bytes < plan->workspace_bytes)
    return fail(GQAP_ERR_INVALID_ARGUMENT, "workspace of %llu bytes < %llu required",
                (unsigned long long)workspace_bytes, (unsigned long long)plan->workspace_bytes);
  if (!std::isfinite(scale) || !std::isfinite(k_scale) || !std::isfinite(v_scale))
    return fail(GQAP_ERR_INVALID_ARGUMENT, "scales must be finite");
  if (d.kv_dtype != GQAP_FP8_E4M3FN && (k_scale != 1.0f || v_scale != 1.0f))
    return fail(GQAP_ERR_INVALID_ARGUMENT, "k_scale/v_scale apply to fp8 KV only and must be 1.0 otherwise");

  const int kv_esz = dtype_size(d.kv_dtype);
  const DecodeWorkspace lay = decode_workspace(d.batch, plan->max_pieces, piece_cols(plan->ratio), d.head_dim);
  char* ws = (char*)workspace;
  DecodeArgs a{};
  a.q = q;
  a.k = k_pool;
  a.v = v_pool;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.prefix = (int32_t*)(ws + lay.prefix);
  a.ws_lse = (float*)(ws + lay.lse);
  a.ws_o = (float*)(ws + lay.o);
  a.out = out;
  a.lse = lse;
  a.q_sb = d.q_stride_batch;
  a.q_sh = d.q_stride_head;
  a.o_sb = d.out_stride_batch;
  a.o_sh = d.out_stride_head;
  a.kv_block_bytes = d.kv_stride_block * kv_esz;
  a.kv_head_bytes = d.kv_stride_head * kv_esz;
  a.bt_stride = d.block_table_stride;
  a.B = d.batch;
  a.Hq = d.num_q_heads;
  a.Hk = d.num_kv_heads;
  a.ratio = plan->ratio;
  a.head_chunks = plan->head_chunks;
  a.hkhc = d.num_kv_heads * plan->head_chunks;
  a.nworkers = plan->num_workers;
  a.pcols = (int32_t)piece_cols(plan->ratio);
  a.max_len = d.max_seq_len;
  a.score_scale = scale * k_scale;
  a.score_scale_log2 = scale * k_scale * dev::kLog2e;
  a.v_scale = v_scale;

  hipStream_t st = (hipStream_t)stream;
  const dim3 grid(plan->num_workers);
  const bool d128 = d.head_dim == 128;
  switch (plan->kernel) {
    case kDecodeF32Valu:
      if (d128)
        hipLaunchKernelGGL(decode_worker_f32<128>, grid, dim3(64), 0, st, a);
      else
        hipLaunchKernelGGL(decode_worker_f32<64>, grid, dim3(64), 0, st, a);
      break;
    case kDecodeBf16Mfma:
      if (d128)
        hipLaunchKernelGGL((decode_worker_mfma<128, false, false>), grid, dim3(64), 0, st, a);
      else
        hipLaunchKernelGGL((decode_worker_mfma<64, false, false>), grid, dim3(64), 0, st, a);
      break;
    case kDecodeFp8Mfma:
      if (d128)
        hipLaunchKernelGGL((decode_worker_mfma<128, true, false>), grid, dim3(64), 0, st, a);
      else
        hipLaunchKernelGGL((decode_worker_mfma<64, true, false>), grid, dim3(64), 0, st, a);
      break;
    default:
      return fail(GQAP_ERR_INVALID_ARGUMENT, "unknown kernel variant %u", plan->kernel);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(GQAP_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
  const dim3 cgrid(d.batch * d.num_q_heads);
  const bool bf16_out = d.q_dtype == GQAP_BF16;
  if (d128) {
    if (bf16_out)
      hipLaunchKernelGGL((decode_combine<128, true, false>), cgrid, dim3(64), 0, st, a);
    else
      hipLaunchKernelGGL((decode_combine<128, false, false>), cgrid, dim3(64), 0, st, a);
  } else {
    if (bf16_out)
      hipLaunchKernelGGL((decode_combine<64, true, false>), cgrid, dim3(64), 0, st, a);
    else
      hipLaunchKernelGGL((decode_combine<64, false, false>), cgrid, dim3(64), 0, st, a);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return fail(GQAP_ERR_HIP, "decode combine launch: %s", hipGetErrorString(e));
  return GQAP_OK;
}

gqap_status gqap::chunk_decode_launch(const gqap_chunk_plan_t* plan, const void* q, const void* k_pool,
                                     const void* v_pool, const void* kr_pool, const int32_t* block_table,
                                     const int32_t* cu_seqlens_q,
                                     const int32_t* kv_lens, float scale, bool fp8, float k_scale, float v_scale,
                                     void* out, float* lse, void* workspace, uint64_t workspace_bytes,
                                     void* stream) {
  const gqap_chunk_desc_t& d = plan->desc;
  if (!workspace) return fail(GQAP_ERR_INVALID_ARGUMENT, "this plan needs a workspace of %llu bytes",
                              (unsigned long long)plan->workspace_bytes);
  if (misaligned(workspace, 256)) return fail(GQAP_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  if (workspace_bytes < plan->workspace_bytes)
    return fail(GQAP_ERR_INVALID_ARGUMENT, "workspace of %llu bytes < %llu required",
                (unsigned long long)workspace_bytes, (unsigned long long)plan->workspace_bytes);
  if (d.head_dim != 128 || (d.head_dim_rope != 0 && d.head_dim_rope != 64) || plan->num_workers <= 0 ||
      plan->head_chunks <= 0)
    return fail(GQAP_ERR_INVALID_ARGUMENT, "chunk plan is not one for the decode workers");
  const bool rope = d.head_dim_rope == 64;
  const int kv_esz = fp8 ? 1 : 2;
  const int64_t pieces = (int64_t)d.batch * d.num_kv_heads * plan->head_chunks + plan->num_workers;
  const int64_t pcols = piece_cols((int64_t)d.max_q_len * plan->ratio);
  const DecodeWorkspace lay = decode_workspace(d.batch, pieces, pcols, d.head_dim);
  if (lay.total > plan->workspace_bytes) return fail(GQAP_ERR_INVALID_ARGUMENT, "chunk plan workspace too small");
  char* ws = (char*)workspace;
  DecodeArgs a{};
  a.q = q;
  a.k = k_pool;
  a.v = v_pool;
  a.block_table = block_table;
  a.seq_lens = kv_lens;
  a.prefix = (int32_t*)(ws + lay.prefix);
  a.ws_lse = (float*)(ws + lay.lse);
  a.ws_o = (float*)(ws + lay.o);
  a.out = out;
  a.lse = lse;
  a.q_sb = d.q_stride_token;
  a.q_sh = d.q_stride_head;
  a.o_sb = d.out_stride_token;
  a.o_sh = d.out_stride_head;
  a.kv_block_bytes = d.kv_stride_block * kv_esz;
  a.kv_head_bytes = d.kv_stride_head * kv_esz;
  a.bt_stride = d.block_table_stride;
  a.B = d.batch;
  a.Hq = d.num_q_heads;
  a.Hk = d.num_kv_heads;
  a.ratio = plan->ratio;
  a.head_chunks = plan->head_chunks;
  a.hkhc = d.num_kv_heads * plan->head_chunks;
  a.nworkers = plan->num_workers;
  a.pcols = (int32_t)pcols;
  a.max_len = d.max_kv_len;
  a.cu = cu_seqlens_q;
  a.max_q = d.max_q_len;
  a.score_scale = scale * (fp8 && !rope ? k_scale : 1.f);
  a.score_scale_log2 = a.score_scale * dev::kLog2e;
  a.v_scale = fp8 ? v_scale : 1.f;
  a.kr = kr_pool;
  a.kr_block_bytes = rope ? d.kr_stride_block * 2 : 0;
  a.nope_scale = fp8 ? k_scale : 1.f;
  hipStream_t st = (hipStream_t)stream;
  if (rope && fp8)
    hipLaunchKernelGGL((decode_worker_rope<true>), dim3(plan->num_workers), dim3(64), 0, st, a);
  else if (rope)
    hipLaunchKernelGGL((decode_worker_rope<false>), dim3(plan->num_workers), dim3(64), 0, st, a);
  else if (fp8)
    hipLaunchKernelGGL((decode_worker_mfma<128, true, true>), dim3(plan->num_workers), dim3(64), 0, st, a);
  else
    hipLaunchKernelGGL((decode_worker_mfma<128, false, true>), dim3(plan->num_workers), dim3(64), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(GQAP_ERR_HIP, "chunk decode launch: %s", hipGetErrorString(e));
  hipLaunchKernelGGL((decode_combine<128, true, true>), dim3(d.batch * d.num_q_heads, d.max_q_len), dim3(64), 0, st,
                     a);
  e = hipGetLastError();
  if (e != hipSuccess) return fail(GQAP_ERR_HIP, "chunk decode combine launch: %s", hipGetErrorString(e));
  return GQAP_OK;
}

extern "C" gqap_status gqap_debug_gather_kv(const gqap_decode_plan_t* plan, const void* pool,
                                            const int32_t* block_table, const int32_t* seq_lens, int32_t b,
                                            int32_t kv_head, int32_t num_rows, void* dst, void* stream) {
  if (!plan || plan->magic != GQAP_PLAN_MAGIC) return fail(GQAP_ERR_INVALID_ARGUMENT, "invalid decode plan");
  const gqap_decode_desc_t& d = plan->desc;
  if (b < 0 || b >= d.batch) return fail(GQAP_ERR_INVALID_ARGUMENT, "b=%d outside [0, %d)", b, d.batch);
  if (kv_head < 0 || kv_head >= d.num_kv_heads)
    return fail(GQAP_ERR_INVALID_ARGUMENT, "kv_head=%d outside [0, %d)", kv_head, d.num_kv_heads);
  if (num_rows < 0 || (int64_t)num_rows > (int64_t)d.max_blocks_per_seq * kBlock)
    return fail(GQAP_ERR_INVALID_ARGUMENT, "num_rows=%d outside [0, Nblk*64]", num_rows);
  if (num_rows == 0) return GQAP_OK;
  if (!pool || !block_table || !seq_lens || !dst) return fail(GQAP_ERR_INVALID_ARGUMENT, "null device pointer");
  if (misaligned(pool, 16) || misaligned(dst, 16))
    return fail(GQAP_ERR_INVALID_ARGUMENT, "pool/dst must be 16-byte aligned");
  const int esz = dtype_size(d.kv_dtype);
  const int row_bytes = d.head_dim * esz;
  const int64_t threads = (int64_t)num_rows * (row_bytes / 16);
  hipLaunchKernelGGL(debug_gather_kv, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, (hipStream_t)stream,
                     (const unsigned char*)pool, block_table, seq_lens, (int64_t)d.block_table_stride,
                     (int64_t)d.kv_stride_block * esz, (int64_t)d.kv_stride_head * esz, row_bytes, b, kv_head,
                     num_rows, (unsigned char*)dst);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(GQAP_ERR_HIP, "gather launch: %s", hipGetErrorString(e));
  return GQAP_OK;
}

extern "C" gqap_status gqap_block_table_from_csr(const int32_t* kv_indices, const int32_t* kv_page_indptr,
                                                 int32_t batch, int32_t max_blocks_per_seq,
                                                 int64_t block_table_stride, int32_t* block_table, void* stream) {
  if (batch < 0) return fail(GQAP_ERR_INVALID_ARGUMENT, "batch must be >= 0");
  if (max_blocks_per_seq < 1) return fail(GQAP_ERR_INVALID_ARGUMENT, "max_blocks_per_seq must be positive");
  if (block_table_stride < max_blocks_per_seq)
    return fail(GQAP_ERR_INVALID_ARGUMENT, "block_table_stride %lld < max_blocks_per_seq %d",
                (long long)block_table_stride, max_blocks_per_seq);
  if (batch == 0) return GQAP_OK;
  if (!kv_indices || !kv_page_indptr || !block_table) return fail(GQAP_ERR_INVALID_ARGUMENT, "null device pointer");
  if (misaligned(kv_indices, 4) || misaligned(kv_page_indptr, 4) || misaligned(block_table, 4))
    return fail(GQAP_ERR_INVALID_ARGUMENT, "index arrays must be 4-byte aligned");
  const int64_t n = (int64_t)batch * max_blocks_per_seq;
  if (n > kMaxLaunchItems) return fail(GQAP_ERR_UNSUPPORTED, "block table of %lld entries too large for one launch",
                                       (long long)n);
  hipLaunchKernelGGL(block_table_from_csr, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, (hipStream_t)stream,
                     kv_indices, kv_page_indptr, batch, max_blocks_per_seq, block_table_stride, block_table);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(GQAP_ERR_HIP, "block_table_from_csr launch: %s", hipGetErrorString(e));
  return GQAP_OK;
}
