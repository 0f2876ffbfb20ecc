// Split-KV paged GQA decode for gfx950.
//
// What is computed (FlashMLA tensor-shape reference, section 1 and the GQA
// diagram): for every sequence b and query head h, attention of the single
// query q[b, h] over the seq_lens[b] keys and values of KV head h / (Hq/Hk),
// gathered block by block through block_table.  MATE's decode path schedules
// the key axis in splits (num_splits); here every split produces a normalised
// partial output and its log-sum-exp, and a second pass merges the splits.
//
// Workgroup (split, kv head, sequence), four waves.  Each wave walks every
// fourth 64-row block of the split with its own online-softmax state; the
// waves are merged through LDS at the end of the split.  Per block:
//   K: global -> registers directly in the matrix-core operand layout;
//   V: global -> registers (contiguous 16-byte chunks) -> LDS (XOR-swizzled)
//      -> transposed LDS reads that deliver the token-packed operand of P.V;
//   S^T = K q^T and O^T += V^T P^T on 16x16x32 bf16 MFMA with fp32 accumulate;
//   the up-to-16 query heads of one KV head share every K/V byte.
#include "dev.hpp"
#include "status.hpp"

#include <cmath>

namespace gqap {

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* block_table;
  const int32_t* seq_lens;
  float* ws_o;    // [B, Hq, S, D] normalised partial outputs
  float* ws_lse;  // [B, Hq, S] partial log-sum-exp, base 2
  void* out;
  float* lse;
  int64_t q_sb, q_sh, o_sb, o_sh;
  int64_t kv_block_bytes, kv_head_bytes, bt_stride;
  int32_t B, Hq, Hk, ratio, head_chunks, nsplit, bps;
  int32_t max_len;         // capacity from the plan; longer seq_lens are clamped to it
  float score_scale_log2;  // scale * k_scale * log2(e)
  float score_scale;       // scale * k_scale
  float v_scale;
};

namespace dev {

// Token (row of the 64-row block) held by MFMA row m of score tile mt.  The
// PV operand needs each 16-lane group to hold 8 tokens that the V transpose
// read delivers: two runs of 4 for 16-bit V, one run of 8 for 8-bit V.
template <bool FP8>
__device__ __forceinline__ int token_of(int mt, int m) {
  if (FP8) return 32 * (mt >> 1) + 8 * (m >> 2) + 4 * (mt & 1) + (m & 3);
  return 16 * mt + m;
}

// Byte offset of (row, byte column c) inside a wave's V tile in LDS.  Rows are
// RB bytes; pieces of P bytes are XOR-permuted within their row so that the
// transpose reads (16 or 32 rows at one column) and the staging stores spread
// over all banks.
template <int RB, int P>
__device__ __forceinline__ int vswz(int row, int c) {
  constexpr int NP = RB / P;
  constexpr int RW = 256 / RB;
  const int piece = (c / P) ^ ((row / RW) % NP);
  return row * RB + piece * P + (c % P);
}

}  // namespace dev

using namespace dev;

template <int D, bool FP8>
__global__ __launch_bounds__(256, 2) void decode_split_mfma(DecodeArgs a) {
  constexpr int ESZ = FP8 ? 1 : 2;
  constexpr int RB = D * ESZ;          // bytes per K/V row
  constexpr int VB = 64 * RB;          // bytes per V slab
  constexpr int PB = FP8 ? 16 : 32;    // swizzle piece
  constexpr int KSTEPS = D / 32;       // MFMA k-steps over the head dim
  constexpr int KLOADS = RB / 64;      // 16-byte loads per row per lane group
  constexpr int NT = D / 16;           // 16-wide output tiles
  constexpr int NV = VB / 1024;        // staging loads per lane
  constexpr int MERGE = 4 * 16 * D * 4 + 2 * 64 * 4;
  constexpr int SMEM = (4 * VB > MERGE) ? 4 * VB : MERGE;
  __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM];

  const int split = blockIdx.x;
  const int g = blockIdx.y / a.head_chunks;
  const int hc = blockIdx.y % a.head_chunks;
  const int b = blockIdx.z;
  const int L = min(max(a.seq_lens[b], 0), a.max_len);
  const int nblk = (L + 63) >> 6;
  const int j0 = split * a.bps;
  if (j0 >= nblk) return;  // the combine pass only reads splits that exist
  const int j1 = min(nblk, j0 + a.bps);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int col = lane & 15;
  const int G = lane >> 4;
  const int hl = hc * 16 + col;
  const bool hvalid = hl < a.ratio;
  const int h = g * a.ratio + hl;

  // Query of head `col` as the B operand; k-slot layout matches the K loads.
  bf16x8 qop[KSTEPS];
  {
    const unsigned char* qp =
        (const unsigned char*)a.q + ((int64_t)b * a.q_sb + (int64_t)(hvalid ? h : 0) * a.q_sh) * 2;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const int d0 = FP8 ? (64 * (ks >> 1) + 16 * G + 8 * (ks & 1)) : (32 * ks + 8 * G);
      i32x4 v = hvalid ? load16(qp + 2 * d0) : i32x4{0, 0, 0, 0};
      qop[ks] = __builtin_bit_cast(bf16x8, v);
    }
  }

  unsigned char* vbuf = smem + wv * VB;
  const unsigned char* kpool = (const unsigned char*)a.k;
  const unsigned char* vpool = (const unsigned char*)a.v;
  const int32_t* bt = a.block_table + (int64_t)b * a.bt_stride;

  float m_run = -INFINITY;
  float l_run = 0.f;
  f32x4 o[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) o[n] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int jb = j0 + wv; jb < j1; jb += 4) {
    const unsigned char* kblk = kv_slab(kpool, bt, jb, g, a.kv_block_bytes, a.kv_head_bytes);
    const unsigned char* vblk = kv_slab(vpool, bt, jb, g, a.kv_block_bytes, a.kv_head_bytes);
    const int valid = min(64, L - jb * 64);

    i32x4 vr[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) vr[i] = load16(vblk + 1024 * i + 16 * lane);
    i32x4 kr[4][KLOADS];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const unsigned char* kp = kblk + token_of<FP8>(mt, col) * RB + 16 * G;
#pragma unroll
      for (int p = 0; p < KLOADS; ++p) kr[mt][p] = load16(kp + 64 * p);
    }

#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int byte = 1024 * i + 16 * lane;
      store16(vbuf + vswz<RB, PB>(byte / RB, byte % RB), vr[i]);
    }

    // S^T[token, head] = K q^T
    f32x4 s[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      s[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        bf16x8 ka;
        if (FP8) {
          const i32x4 w = kr[mt][ks >> 1];
          ka = fp8x8_to_bf16x8(i32x2{w[2 * (ks & 1)], w[2 * (ks & 1) + 1]});
        } else {
          ka = __builtin_bit_cast(bf16x8, kr[mt][ks]);
        }
        s[mt] = mfma16x16x32(ka, qop[ks], s[mt]);
      }
    }

    // Online softmax in base 2.  Keys past seq_len are dropped by select, so
    // whatever the padding rows hold never reaches the sums.
    float bmax = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float x = token_of<FP8>(mt, 4 * G + j) < valid ? s[mt][j] * a.score_scale_log2 : -INFINITY;
        s[mt][j] = x;
        bmax = fmaxf(bmax, x);
      }
    bmax = fmaxf(bmax, __shfl_xor(bmax, 16));
    bmax = fmaxf(bmax, __shfl_xor(bmax, 32));
    const float m_new = fmaxf(m_run, bmax);
    const float alpha = exp2f(m_run - m_new);
    float psum = 0.f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p = exp2f(s[mt][j] - m_new);
        s[mt][j] = p;
        psum += p;
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int n = 0; n < NT; ++n) o[n] *= alpha;

    // P^T as the B operand: k-slot e of lane group G is token_of(2ks + e/4, 4G + e%4).
    bf16x8 pop[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      i32x4 w;
      w[0] = (int)pack_bf16x2(s[2 * ks][0], s[2 * ks][1]);
      w[1] = (int)pack_bf16x2(s[2 * ks][2], s[2 * ks][3]);
      w[2] = (int)pack_bf16x2(s[2 * ks + 1][0], s[2 * ks + 1][1]);
      w[3] = (int)pack_bf16x2(s[2 * ks + 1][2], s[2 * ks + 1][3]);
      pop[ks] = __builtin_bit_cast(bf16x8, w);
    }

    lds_fence();  // this wave's V tile is in LDS

    // O^T[d, head] += V^T P^T
#pragma unroll
    for (int n = 0; n < NT; ++n) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        bf16x8 va;
        if (FP8) {
          const int t0 = 32 * ks + 8 * G;
          i32x2 w = lds_read_tr8(vbuf + vswz<RB, PB>(t0 + (col >> 1), 16 * n + 8 * (col & 1)));
          if (valid < 64) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (t0 + e >= valid) w[e >> 2] &= ~(0xff << (8 * (e & 3)));
          }
          va = fp8x8_to_bf16x8(w);
        } else {
          i32x4 w;
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const int t0 = 32 * ks + 16 * half + 4 * G;
            const i16x4 r = lds_read_tr16(vbuf + vswz<RB, PB>(t0 + (col >> 2), 32 * n + 8 * (col & 3)));
            uint32_t lo = (uint16_t)r[0] | ((uint32_t)(uint16_t)r[1] << 16);
            uint32_t hi = (uint16_t)r[2] | ((uint32_t)(uint16_t)r[3] << 16);
            if (valid < 64) {
              if (t0 + 0 >= valid) lo &= 0xffff0000u;
              if (t0 + 1 >= valid) lo &= 0x0000ffffu;
              if (t0 + 2 >= valid) hi &= 0xffff0000u;
              if (t0 + 3 >= valid) hi &= 0x0000ffffu;
            }
            w[2 * half] = (int)lo;
            w[2 * half + 1] = (int)hi;
          }
          va = __builtin_bit_cast(bf16x8, w);
        }
        o[n] = mfma16x16x32(va, pop[ks], o[n]);
      }
    }
  }

  // Merge the four waves of this split.
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  __syncthreads();  // every wave is done with its V tile
  float* sO = (float*)smem;             // [4 waves][16 heads][D]
  float* sM = sO + 4 * 16 * D;          // [4][16]
  float* sL = sM + 64;                  // [4][16]
#pragma unroll
  for (int n = 0; n < NT; ++n)
#pragma unroll
    for (int j = 0; j < 4; ++j) sO[(wv * 16 + col) * D + 16 * n + 4 * G + j] = o[n][j];
  if (G == 0) {
    sM[wv * 16 + col] = m_run;
    sL[wv * 16 + col] = l_tot;
  }
  __syncthreads();
  const int rc = min(16, a.ratio - hc * 16);
  for (int idx = tid; idx < rc * D; idx += 256) {
    const int hh = idx / D;
    const int d = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sM[w * 16 + hh]);
    float den = 0.f, num = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float wt = exp2f(sM[w * 16 + hh] - M);
      den += sL[w * 16 + hh] * wt;
      num += sO[(w * 16 + hh) * D + d] * wt;
    }
    const int hq = g * a.ratio + hc * 16 + hh;
    const int64_t row = ((int64_t)b * a.Hq + hq) * a.nsplit + split;
    a.ws_o[row * D + d] = num / den * a.v_scale;
    if (d == 0) a.ws_lse[row] = M + log2f(den);
  }
}

// fp32 path: one wave per (split, kv head, sequence, head chunk), vector ALU.
// Lane t scores token t of a block (K staged in LDS); lane d accumulates
// output columns d, d+64 reading V rows straight from the pool (rows past
// seq_len are never touched).
template <int D>
__global__ __launch_bounds__(64) void decode_split_f32(DecodeArgs a) {
  constexpr int DC = D / 64;
  __shared__ float sK[64][D + 1];
  __shared__ float sQ[16][D];
  __shared__ float sP[16][64];

  const int split = blockIdx.x;
  const int g = blockIdx.y / a.head_chunks;
  const int hc = blockIdx.y % a.head_chunks;
  const int b = blockIdx.z;
  const int L = min(max(a.seq_lens[b], 0), a.max_len);
  const int nblk = (L + 63) >> 6;
  const int j0 = split * a.bps;
  if (j0 >= nblk) return;
  const int j1 = min(nblk, j0 + a.bps);
  const int lane = threadIdx.x;
  const int rc = min(16, a.ratio - hc * 16);
  const int hbase = g * a.ratio + hc * 16;

  const float* q = (const float*)a.q;
  for (int i = lane; i < 16 * D; i += 64) {
    const int hh = i / D, d = i % D;
    sQ[hh][d] = hh < rc ? q[(int64_t)b * a.q_sb + (int64_t)(hbase + hh) * a.q_sh + d] : 0.f;
  }
  float m[16], l[16], o[16][DC];
#pragma unroll
  for (int hh = 0; hh < 16; ++hh) {
    m[hh] = -INFINITY;
    l[hh] = 0.f;
#pragma unroll
    for (int c = 0; c < DC; ++c) o[hh][c] = 0.f;
  }
  const unsigned char* kpool = (const unsigned char*)a.k;
  const unsigned char* vpool = (const unsigned char*)a.v;
  const int32_t* bt = a.block_table + (int64_t)b * a.bt_stride;

  for (int jb = j0; jb < j1; ++jb) {
    const float* kblk = (const float*)kv_slab(kpool, bt, jb, g, a.kv_block_bytes, a.kv_head_bytes);
    const float* vblk = (const float*)kv_slab(vpool, bt, jb, g, a.kv_block_bytes, a.kv_head_bytes);
    const int valid = min(64, L - jb * 64);
    __syncthreads();
    for (int i = lane; i < 64 * D; i += 64) {
      const int t = i / D, d = i % D;
      sK[t][d] = t < valid ? kblk[i] : 0.f;
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
      for (int off = 32; off > 0; off >>= 1) bmax = fmaxf(bmax, __shfl_xor(bmax, off));
      const float m_new = fmaxf(m[hh], bmax);
      const float alpha = expf(m[hh] - m_new);
      const float p = lane < valid ? expf(sc - m_new) : 0.f;
      float ps = p;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) ps += __shfl_xor(ps, off);
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
  }
#pragma unroll
  for (int hh = 0; hh < 16; ++hh) {
    if (hh >= rc) break;
    const int64_t row = ((int64_t)b * a.Hq + hbase + hh) * a.nsplit + split;
#pragma unroll
    for (int c = 0; c < DC; ++c) a.ws_o[row * D + lane + 64 * c] = o[hh][c] / l[hh] * a.v_scale;
    if (lane == 0) a.ws_lse[row] = m[hh] * kLog2e + log2f(l[hh]);
  }
}

// Merge the splits of one (sequence, query head): weights 2^(lse_s - max).
template <int D, bool OUT_BF16>
__global__ __launch_bounds__(64) void decode_combine(DecodeArgs a) {
  constexpr int DC = D / 64;
  const int bh = blockIdx.x;
  const int b = bh / a.Hq;
  const int h = bh % a.Hq;
  const int lane = threadIdx.x;
  const int L = min(max(a.seq_lens[b], 0), a.max_len);
  const int nblk = (L + 63) >> 6;
  const int ns = (nblk + a.bps - 1) / a.bps;
  const float* lse2 = a.ws_lse + (int64_t)bh * a.nsplit;
  const float* op = a.ws_o + (int64_t)bh * a.nsplit * D;
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, lse2[s]);
  float den = 0.f;
  float acc[DC];
#pragma unroll
  for (int c = 0; c < DC; ++c) acc[c] = 0.f;
  for (int s = 0; s < ns; ++s) {
    const float w = exp2f(lse2[s] - M);
    den += w;
#pragma unroll
    for (int c = 0; c < DC; ++c) acc[c] = fmaf(w, op[(int64_t)s * D + lane + 64 * c], acc[c]);
  }
  const int64_t obase = (int64_t)b * a.o_sb + (int64_t)h * a.o_sh;
#pragma unroll
  for (int c = 0; c < DC; ++c) {
    const float v = ns > 0 ? acc[c] / den : 0.f;
    if (OUT_BF16)
      ((uint16_t*)a.out)[obase + lane + 64 * c] = f32_to_bf16(v);
    else
      ((float*)a.out)[obase + lane + 64 * c] = v;
  }
  if (a.lse && lane == 0) a.lse[bh] = ns > 0 ? (M + log2f(den)) * kLn2 : -INFINITY;
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

}  // namespace gqap

using namespace gqap;

extern "C" gqap_status gqap_paged_decode(const gqap_decode_plan_t* plan, const void* q, const void* k_pool,
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
  DecodeArgs a{};
  a.q = q;
  a.k = k_pool;
  a.v = v_pool;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  const int64_t rows = (int64_t)d.batch * d.num_q_heads * plan->num_splits;
  a.ws_o = (float*)workspace;
  a.ws_lse = (float*)((char*)workspace + ((rows * d.head_dim * 4 + 255) & ~int64_t(255)));
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
  a.nsplit = plan->num_splits;
  a.bps = plan->blocks_per_split;
  a.max_len = d.max_seq_len;
  a.score_scale = scale * k_scale;
  a.score_scale_log2 = scale * k_scale * dev::kLog2e;
  a.v_scale = v_scale;

  hipStream_t st = (hipStream_t)stream;
  const dim3 grid(plan->num_splits, d.num_kv_heads * plan->head_chunks, d.batch);
  const bool d128 = d.head_dim == 128;
  switch (plan->kernel) {
    case kDecodeF32Valu:
      if (d128)
        hipLaunchKernelGGL(decode_split_f32<128>, grid, dim3(64), 0, st, a);
      else
        hipLaunchKernelGGL(decode_split_f32<64>, grid, dim3(64), 0, st, a);
      break;
    case kDecodeBf16Mfma:
      if (d128)
        hipLaunchKernelGGL((decode_split_mfma<128, false>), grid, dim3(256), 0, st, a);
      else
        hipLaunchKernelGGL((decode_split_mfma<64, false>), grid, dim3(256), 0, st, a);
      break;
    case kDecodeFp8Mfma:
      if (d128)
        hipLaunchKernelGGL((decode_split_mfma<128, true>), grid, dim3(256), 0, st, a);
      else
        hipLaunchKernelGGL((decode_split_mfma<64, true>), grid, dim3(256), 0, st, a);
      break;
    default:
      return fail(GQAP_ERR_INVALID_ARGUMENT, "unknown kernel variant %u", plan->kernel);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(GQAP_ERR_HIP, "decode split launch: %s", hipGetErrorString(e));
  const dim3 cgrid(d.batch * d.num_q_heads);
  const bool bf16_out = d.q_dtype == GQAP_BF16;
  if (d128) {
    if (bf16_out)
      hipLaunchKernelGGL((decode_combine<128, true>), cgrid, dim3(64), 0, st, a);
    else
      hipLaunchKernelGGL((decode_combine<128, false>), cgrid, dim3(64), 0, st, a);
  } else {
    if (bf16_out)
      hipLaunchKernelGGL((decode_combine<64, true>), cgrid, dim3(64), 0, st, a);
    else
      hipLaunchKernelGGL((decode_combine<64, false>), cgrid, dim3(64), 0, st, a);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return fail(GQAP_ERR_HIP, "decode combine launch: %s", hipGetErrorString(e));
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
  if (misaligned(pool, 16) || misaligned(dst, 16)) return fail(GQAP_ERR_INVALID_ARGUMENT, "pool/dst must be 16-byte aligned");
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
