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
// query tile); each wave owns 32 query rows.  Key tiles of 64 rows (K, the
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

#include <cmath>

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
  float scale_log2;  // scale * log2(e)
};

namespace dev {

typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

__device__ __forceinline__ f32x16_t mfma32x32x16(bf16x8 a, bf16x8 b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
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

// V tile (64 rows x 256 bytes): 32-byte pieces permuted by row, for the
// transpose reads (4 rows x 32 bytes per 16 lanes).
__device__ __forceinline__ int vswz256(int row, int c) {
  return row * 256 + ((((c >> 5) ^ (row & 7))) << 5) + (c & 31);
}

}  // namespace dev

using namespace dev;

template <int DR>
__global__ __launch_bounds__(256, 2) void prefill_fwd(PrefillArgs a) {
  constexpr int DN = 128;                 // per-head key width
  constexpr int DV = 128;                 // value / output width
  constexpr int KSN = DN / 16;            // k-steps over the nope part
  constexpr int KSR = DR / 16;            // k-steps over the rope part
  constexpr int KB = 64 * DN * 2;         // K tile bytes
  constexpr int RB = 64 * (DR ? DR : 8) * 2;  // rope tile bytes (unused when DR == 0)
  constexpr int VB = 64 * DV * 2;         // V tile bytes
  constexpr int STAGE = KB + (DR ? RB : 0) + VB;
  constexpr int KLD = KB / 16 / 256;      // 16-byte staging loads per thread: K
  constexpr int RLD = DR ? RB / 16 / 256 : 0;
  constexpr int VLD = VB / 16 / 256;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * STAGE];

  // Work item: deepest query tile first; heads of one KV group on one XCD.
  const int x = blockIdx.x;                   // 0 .. Hq-1
  const int hpx = a.Hq >> 3;                  // heads per XCD slot (Hq % 8 == 0), else identity
  const int h = (a.Hq & 7) ? x : (x & 7) * hpx + (x >> 3);
  const int b = blockIdx.y;
  const int qt = a.q_tiles - 1 - (int)blockIdx.z;
  const int c0 = a.cu[b];
  const int L = min(a.cu[b + 1] - c0, a.max_len);  // capacity from the plan
  const int q0 = qt * 128;
  if (q0 >= L) return;
  const int g = h / a.ratio;

  const int tid = threadIdx.x;
  const int wv = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int r0 = q0 + 32 * wv;               // first query row of this wave (local)
  const int qrow = r0 + l32;                 // this lane's query row
  const bool wave_rows = r0 < L;
  const int rlast = min(L, r0 + 32) - 1;     // last valid row of the wave

  // The wave's queries as the B operand: lane (query l32, half hh) holds
  // d = 16 s + 8 hh .. +7 for k-step s (s < KSN: nope part, then rope).
  bf16x8 qop[KSN + KSR];
  {
    const bool ok = qrow < L;
    const uint16_t* qp = a.q + (int64_t)(c0 + (ok ? qrow : 0)) * a.q_st + (int64_t)h * a.q_sh;
#pragma unroll
    for (int s = 0; s < KSN + KSR; ++s) {
      const i32x4 v = ok ? load16(qp + 16 * s + 8 * hh) : i32x4{0, 0, 0, 0};
      qop[s] = __builtin_bit_cast(bf16x8, v);
    }
  }

  // Key tiles this workgroup must visit: keys < min(L, q0 + 128).
  const int nkt = (min(L, q0 + 128) + 63) >> 6;
  const int qb0 = q0 >> 6;                   // the workgroup's two query blocks
  const int qb1 = min(qb0 + 1, (L - 1) >> 6);
  const uint8_t* mrow0 = a.mask ? a.mask + ((int64_t)b * a.mask_nb + qb0) * a.mask_nb : nullptr;
  const uint8_t* mrow1 = a.mask ? a.mask + ((int64_t)b * a.mask_nb + qb1) * a.mask_nb : nullptr;
  // A key tile is needed if either query block sees it (causal order first).
  auto tile_needed = [&](int kt) {
    if (!a.mask) return true;
    const bool v0 = kt <= qb0 && mrow0[kt];
    const bool v1 = kt <= qb1 && mrow1[kt];
    return v0 || v1;
  };
  auto next_tile = [&](int kt) {
    ++kt;
    while (kt < nkt && !tile_needed(kt)) ++kt;
    return kt;
  };
  const int wqb = r0 >> 6;                   // this wave's query block
  const uint8_t* mroww = a.mask ? a.mask + ((int64_t)b * a.mask_nb + wqb) * a.mask_nb : nullptr;

  // Staging: thread tid moves chunks tid + 256 i of each tile.
  i32x4 kst[KLD], rst[RLD > 0 ? RLD : 1], vst[VLD];
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int i = 0; i < KLD; ++i) {
      const int chunk = tid + 256 * i;
      const int row = chunk >> 4, c = chunk & 15;
      const int key = kt * 64 + row;
      kst[i] = key < L ? load16(a.k + (int64_t)(c0 + key) * a.k_st + (int64_t)g * a.k_sh + 8 * c)
                       : i32x4{0, 0, 0, 0};
    }
    if constexpr (DR > 0) {
#pragma unroll
      for (int i = 0; i < RLD; ++i) {
        const int chunk = tid + 256 * i;
        const int row = chunk >> 3, c = chunk & 7;
        const int key = kt * 64 + row;
        rst[i] = key < L ? load16(a.kr + (int64_t)(c0 + key) * a.kr_st + 8 * c) : i32x4{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int i = 0; i < VLD; ++i) {
      const int chunk = tid + 256 * i;
      const int row = chunk >> 4, c = chunk & 15;
      const int key = kt * 64 + row;
      vst[i] = key < L ? load16(a.v + (int64_t)(c0 + key) * a.v_st + (int64_t)g * a.v_sh + 8 * c)
                       : i32x4{0, 0, 0, 0};
    }
  };
  auto store_tile = [&](int buf) {
    unsigned char* st = smem + buf * STAGE;
#pragma unroll
    for (int i = 0; i < KLD; ++i) {
      const int chunk = tid + 256 * i;
      store16(st + kswz<16>(chunk >> 4, chunk & 15), kst[i]);
    }
    if constexpr (DR > 0) {
#pragma unroll
      for (int i = 0; i < RLD; ++i) {
        const int chunk = tid + 256 * i;
        store16(st + KB + kswz<8>(chunk >> 3, chunk & 7), rst[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < VLD; ++i) {
      const int chunk = tid + 256 * i;
      store16(st + KB + (DR ? RB : 0) + vswz256(chunk >> 4, (chunk & 15) << 4), vst[i]);
    }
  };

  float m_run = -INFINITY, l_run = 0.f;  // per query (both halves of a query agree)
  f32x16_t o[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) o[t] = f32x16_t{};

  auto compute_tile = [&](int kt, int buf) {
    const unsigned char* st = smem + buf * STAGE;
    // S^T tile t (keys 32t .. 32t+31 of the tile) x 32 queries.
    f32x16_t s[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      s[t] = f32x16_t{};
      const int krow = 32 * t + l32;
#pragma unroll
      for (int ss = 0; ss < KSN; ++ss) {
        const bf16x8 ka = __builtin_bit_cast(bf16x8, load16(st + kswz<16>(krow, 2 * ss + hh)));
        s[t] = mfma32x32x16(ka, qop[ss], s[t]);
      }
      if constexpr (DR > 0) {
#pragma unroll
        for (int ss = 0; ss < KSR; ++ss) {
          const bf16x8 ka = __builtin_bit_cast(bf16x8, load16(st + KB + kswz<8>(krow, 2 * ss + hh)));
          s[t] = mfma32x32x16(ka, qop[KSN + ss], s[t]);
        }
      }
    }
    // Scale, mask (causal, ragged end) by select, running max.
    const bool need_mask = kt * 64 + 63 > r0;  // tile reaches past this wave's first row
    float tmax = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        float x = s[t][j] * a.scale_log2;
        if (need_mask) {
          const int key = kt * 64 + 32 * t + (j >> 2) * 8 + hh * 4 + (j & 3);
          x = key <= qrow ? x : -INFINITY;
        }
        s[t][j] = x;
        tmax = fmaxf(tmax, x);
      }
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, tmax),
                                                       __builtin_bit_cast(uint32_t, tmax), false, false);
      tmax = fmaxf(__builtin_bit_cast(float, (uint32_t)sw[0]), __builtin_bit_cast(float, (uint32_t)sw[1]));
    }
    const float m_new = fmaxf(m_run, tmax);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;  // a row with nothing visible yet
    const float alpha = fast_exp2(m_run - m_use);
    float psum = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float p = fast_exp2(s[t][j] - m_use);
        s[t][j] = p;
        psum += p;
      }
    l_run = l_run * alpha + psum;  // this lane's half of the row sum
    m_run = m_new;
#pragma unroll
    for (int t = 0; t < 4; ++t) o[t] *= alpha;
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
    // O^T[d, q] += V^T P^T.  16-lane group gamma reads d = 32 dt + 16 (gamma & 1) + i
    // at keys kb .. kb+3 through the transpose read.
    const unsigned char* vt = st + KB + (DR ? RB : 0);
    const int gam = lane >> 4;
    const int li = lane & 15;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const int db = 32 * dt + 16 * (gam & 1);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        i32x4 w;
#pragma unroll
        for (int part = 0; part < 2; ++part) {
          const int kb = 16 * ks + 8 * part + 4 * hh;
          const i16x4 r = lds_read_tr16(vt + vswz256(kb + (li >> 2), 2 * (db + 4 * (li & 3))));
          w[2 * part] = (int)((uint16_t)r[0] | ((uint32_t)(uint16_t)r[1] << 16));
          w[2 * part + 1] = (int)((uint16_t)r[2] | ((uint32_t)(uint16_t)r[3] << 16));
        }
        o[dt] = mfma32x32x16(__builtin_bit_cast(bf16x8, w), pop[ks], o[dt]);
      }
    }
  };

  // A wave computes a loaded tile only if its own rows see some key of it.
  auto wave_sees = [&](int kt) {
    if (!wave_rows || kt * 64 > rlast) return false;
    return !a.mask || mroww[kt];
  };

  int kt = tile_needed(0) ? 0 : next_tile(0);
  int buf = 0;
  if (kt < nkt) {
    load_tile(kt);
    store_tile(0);
  }
  __syncthreads();
  while (kt < nkt) {
    const int kn = next_tile(kt);
    if (kn < nkt) load_tile(kn);
    if (wave_sees(kt)) compute_tile(kt, buf);
    if (kn < nkt) store_tile(buf ^ 1);
    __syncthreads();
    kt = kn;
    buf ^= 1;
  }

  // Epilogue: combine the two halves of each row sum, normalise, store.
  if (!wave_rows) return;
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, l_run),
                                                     __builtin_bit_cast(uint32_t, l_run), false, false);
    l_run = __builtin_bit_cast(float, (uint32_t)sw[0]) + __builtin_bit_cast(float, (uint32_t)sw[1]);
  }
  if (qrow >= L) return;
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
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

static bool misaligned16(const void* p) { return ((uintptr_t)p) & 15; }

}  // namespace gqap

using namespace gqap;

extern "C" gqap_status gqap_prefill(const gqap_prefill_plan_t* plan, const void* q, const void* k, const void* v,
                                    const void* k_rope, const int32_t* cu_seqlens, const uint8_t* block_mask,
                                    float scale, void* out, float* lse, void* workspace, uint64_t workspace_bytes,
                                    void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  if (!plan || plan->magic != GQAP_PLAN_MAGIC) return fail(GQAP_ERR_INVALID_ARGUMENT, "invalid prefill plan");
  const gqap_prefill_desc_t& d = plan->desc;
  if (d.batch == 0 || plan->q_tiles == 0) return GQAP_OK;
  if (!q || !k || !v || !cu_seqlens || !out) return fail(GQAP_ERR_INVALID_ARGUMENT, "null device pointer");
  if (d.head_dim_rope && !k_rope) return fail(GQAP_ERR_INVALID_ARGUMENT, "k_rope is required when head_dim_rope > 0");
  if (!d.head_dim_rope && k_rope) return fail(GQAP_ERR_INVALID_ARGUMENT, "k_rope given but head_dim_rope == 0");
  if (d.has_block_mask && !block_mask) return fail(GQAP_ERR_INVALID_ARGUMENT, "block mask declared but null");
  if (misaligned16(q) || misaligned16(k) || misaligned16(v) || misaligned16(out) ||
      (k_rope && misaligned16(k_rope)) || ((uintptr_t)cu_seqlens & 3) || (lse && ((uintptr_t)lse & 3)))
    return fail(GQAP_ERR_INVALID_ARGUMENT, "device pointers must be 16-byte aligned (cu_seqlens, lse 4-byte)");
  if (!std::isfinite(scale)) return fail(GQAP_ERR_INVALID_ARGUMENT, "scale must be finite");
  PrefillArgs a{};
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.kr = (const uint16_t*)k_rope;
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
  a.mask_nb = d.mask_blocks;
  a.max_len = d.max_seq_len;
  a.scale_log2 = scale * dev::kLog2e;
  const dim3 grid(d.num_q_heads, d.batch, plan->q_tiles);
  hipStream_t st = (hipStream_t)stream;
  if (d.head_dim_rope == 64)
    hipLaunchKernelGGL(prefill_fwd<64>, grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(prefill_fwd<0>, grid, dim3(256), 0, st, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(GQAP_ERR_HIP, "prefill launch: %s", hipGetErrorString(e));
  return GQAP_OK;
}
