// Multi-query attention over quantized pages with both contractions on
// v_mfma_f32_16x16x32_f16, 16 (query, head) rows per MFMA: the read path of
// a speculative verify or a prefill chunk, where the n_q newest cached
// tokens of a sequence attend causally to the tokens up to their own
// positions, straight from the compressed pages (aitrends.kr article 74976,
// TL;DR: the attention backend reads compressed KV pages without
// re-materializing fp16 K/V).
//
// The algebra is the decode kernel's (kvq_decode_kernel.h): scores are
// S_t sum_c qt_c k_tc + O_t sum_c qt_c with qt = (H q) * alpha_K folded once
// per tile, and values accumulate alpha_V (sum_t p_t S_t k_tc + sum_t p_t O_t)
// in the rotated basis; the partition merge applies the final H.
//
// Work split: one workgroup of 4 waves per (sequence, kv head, block of up to
// 64 rows, partition of 64-token chunks).  A wave owns a tile of 16 rows and
// walks the partition's chunks (with fewer than 4 row tiles, the waves of a
// row tile take every 4 / tiles-th chunk); the pages are read once per
// workgroup, each wave reading them for its own rows (the second read is
// served from cache).
//
// Lane layouts (lane l: n = l mod 16, g = l / 16):
//   QK   D[token][row] = sum_k K[token][k] qt[row][k]: A = the codes of token
//        n of a 16-token page, B = the folded query of row n; lane group g
//        supplies code block g of its token (units 4 g .. 4 g + 3, one unit
//        per 32-wide k step) and the matching 8 query channels.  Output: lane
//        holds row n and tokens 4 g + i (i < 4) of the page.
//   PV   D[row][channel] = sum_k P[row][k] V[k][channel]: A = the
//        probabilities of row n for the lane's own tokens 4 g + i of two
//        pages (no transpose: the QK output already sits there), B = the V
//        codes of channel n (+ 16 j) for the same tokens, read from the V
//        runs (one word per token quad and run).  Output: lane holds channel
//        16 j + n and rows 4 g + i.
// Codes enter as fp16 denormals as in the decode kernel; operands are split
// hi / lo on the same exact grids, so the hi chains sum exactly.
#pragma once
#include "kvq_decode_kernel.h"

namespace kvq {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kMqBlockRows = 64;   // rows per workgroup (4 tiles of 16)

__device__ __forceinline__ f16x8 as_f16x8(unsigned a, unsigned b, unsigned c, unsigned d) {
  return __builtin_bit_cast(f16x8, u32x4{a, b, c, d});
}
__device__ __forceinline__ f32x4 mfma16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Channel of QK k step ks (< 4), operand element e (< 8) for lane group g:
// 16 m + 4 g + j with (m, j) below.  The elements follow the code fields as
// one unit (4 and 8 bits) or two units (2 bits) unpack into 8 halves:
//   4 bits: unit 4 g + ks, halves f0 f4 f1 f5 f2 f6 f3 f7
//   8 bits: unit 4 g + ks, halves f0 f2 f1 f3 f4 f6 f5 f7
//   2 bits: units 4 g + 2 (ks / 2) + {0, 1}, fields 4 (ks % 2) + {0..3},
//           halves (unit 0, unit 1) per field.
template <int BITS>
__host__ __device__ constexpr int mq_field(int ks, int e) {
  if constexpr (BITS == 4) return (e >> 1) + 4 * (e & 1);
  else if constexpr (BITS == 8) return 4 * (e >> 2) + ((e & 1) << 1) + ((e >> 1) & 1);
  else return 4 * (ks & 1) + (e >> 1);
}
template <int BITS>
__host__ __device__ constexpr int mq_off(int ks, int e) {
  if constexpr (BITS == 2) return 2 * (ks >> 1) + (e & 1);
  else return ks;
}

// QK A operand of k step ks from the lane's code block (4 units)
template <int BITS, int NB>
__device__ __forceinline__ f16x8 mq_k_operand(const u32x4 (&blk)[NB], int ks) {
  if constexpr (BITS == 4) {
    const unsigned x = blk[0][ks], y = x >> 8;
    return as_f16x8(x & 0x000F000Fu, x & 0x00F000F0u, y & 0x000F000Fu, y & 0x00F000F0u);
  } else if constexpr (BITS == 8) {
    const unsigned a = blk[(ks >> 1) % NB][2 * (ks & 1)], b = blk[(ks >> 1) % NB][2 * (ks & 1) + 1];
    return as_f16x8(a & 0x00FF00FFu, (a >> 8) & 0x00FF00FFu, b & 0x00FF00FFu, (b >> 8) & 0x00FF00FFu);
  } else {
    const unsigned x = (ks & 1) ? (blk[0][ks >> 1] >> 8) : blk[0][ks >> 1];
    return as_f16x8(x & 0x00030003u, x & 0x000C000Cu, x & 0x00300030u, x & 0x00C000C0u);
  }
}

// PV B operand halves (2 words = 4 tokens of one quad) of channel half h
// from the quad's word(s) of a V run; x2 is the second word at 8 bits
template <int BITS>
__device__ __forceinline__ void mq_v_fields(unsigned x, unsigned x2, int h, unsigned& a, unsigned& b) {
  if constexpr (BITS == 4) {
    const unsigned z = h ? (x >> 8) : x;
    a = z & 0x000F000Fu;
    b = z & 0x00F000F0u;
  } else if constexpr (BITS == 8) {
    const unsigned z = h ? x2 : x;
    a = z & 0x00FF00FFu;
    b = (z >> 8) & 0x00FF00FFu;
  } else {
    a = x & (h ? 0x00300030u : 0x00030003u);
    b = x & (h ? 0x00C000C0u : 0x000C000Cu);
  }
}

template <int BITS, bool M16>
__device__ __forceinline__ f32x4 load_meta4(const uint8_t* p, int i) {   // elements i .. i + 3
  if constexpr (M16) {
    const u32x2 w = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p + 2 * i));
    return f32x4{half_bits_to_float((uint16_t)w[0]), half_bits_to_float((uint16_t)(w[0] >> 16)),
                 half_bits_to_float((uint16_t)w[1]), half_bits_to_float((uint16_t)(w[1] >> 16))};
  } else {
    return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + 4 * i));
  }
}

struct alignas(16) MqSmem {
  const __attribute__((address_space(1))) uint8_t* kp[kSlotEntries];
  const __attribute__((address_space(1))) uint8_t* vp[kSlotEntries];
  float meta[kWaves][4 * kChunk];   // per wave: the chunk's S_K, O_K, S_V, O_V by token
  union {
    float hq[kMqBlockRows][kHeadDim];   // (H q)_c / (weight of c's K field) per row
    struct {
      float acc[kWaves][16][kHeadDim];
      float m[kWaves][16];
      float l[kWaves][16];
    } merge;
  };
};

template <int T, int BK, int BV, bool M16, bool KCH>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu((T != 32 && BK != 8 && BV != 8) ? 2 : 1))) void mq_dense_kernel(DecodeArgs A) {
  constexpr int SLOT_K = slot_bytes(BK, T, M16, KCH), SLOT_V = slot_bytes(BV, T, M16);
  constexpr int CODE_K = slot_code_bytes(BK), CODE_V = slot_code_bytes(BV);
  constexpr int OFF_K = slot_offset_at(BK, M16), OFF_V = slot_offset_at(BV, M16);
  // KCH (K rounded per channel): the fold takes the channel scales A, both
  // per-token factors are beta, and the offset term is sum_c qt_c M_c
  constexpr int ALPHA_K = KCH ? slot_chan_scale_at(BK) : slot_alpha_at(BK, M16), ALPHA_V = slot_alpha_at(BV, M16);
  constexpr int ZP_K = slot_chan_zp_at(BK, T);
  constexpr int AL = slot_alpha_len(T);   // channels of a tile's alpha per page
  constexpr int PPT = T / kPage;
  // V tokens 2, 3 of a quad weigh kTok times tokens 0, 1 (their probabilities
  // enter divided by kTok); at 2 bits channel half 1 weighs 16 times half 0
  constexpr float kTok = (BV == 8) ? 1.f : (BV == 4) ? 16.f : 4.f;
  constexpr int QE = (BK == 8) ? 6 : 10, PE = (BV == 8) ? 6 : 10;
  constexpr float kTwo24 = 16777216.f;
  __shared__ MqSmem sm;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, g = lane >> 4;
  const int H = A.kv_heads, G = A.group;
  const int rows = A.n_q * G;
  const int RB = (rows + kMqBlockRows - 1) / kMqBlockRows;
  const int part = blockIdx.y;
  const int seq = (int)blockIdx.x / (H * RB);
  const int hb = (int)blockIdx.x - seq * H * RB;
  const int kvh = hb % H;
  const int r0 = (hb / H) * kMqBlockRows;
  const int nrows = min(kMqBlockRows, rows - r0);
  const int nrt = (nrows + 15) / 16;             // row tiles (1..4)
  const int nsub = kWaves / nrt;                 // waves per row tile
  const int rt = wave % nrt, sub = wave / nrt;   // uniform
  const bool active = sub < nsub;
  const int L = A.seq_lens[seq];
  const int nchunks = min((L + kChunk - 1) / kChunk, A.max_tiles);
  const int c_begin = part * A.tiles_per_part;
  const int c_end = min(nchunks, c_begin + A.tiles_per_part);
  if (c_begin >= c_end) return;   // uniform over the workgroup

  // the row tile's queries (the waves that compute H q), loaded first
  const bool hq_wave = wave < nrt;
  const int my_row = r0 + 16 * rt + n;            // QK-side row of this lane
  const bool row_real = 16 * rt + n < nrows;
  u32x4 qraw[4];
  if (hq_wave) {
    const int r = row_real ? my_row : r0;
    const size_t qix = ((size_t)seq * A.n_q + r / G) * A.q_heads + kvh * G + r % G;
    const uint16_t* qrow = A.q + qix * kHeadDim + 32 * g;
#pragma unroll
    for (int v = 0; v < 4; ++v) qraw[v] = *reinterpret_cast<const u32x4*>(qrow + 8 * v);   // (zeroed at use past the real rows)
  }
  // the partition's slots
  const int npages = ((L + T - 1) / T) * PPT;
  {
    const int32_t* trow = A.block_table + (size_t)seq * A.max_blocks + 4 * c_begin;
    const int last = min(npages, ((4 * c_end + PPT - 1) / PPT) * PPT);
    const int np = last - 4 * c_begin;
    // (entries past the partition's pages point at the spare slot: the loads
    // issued after a wave's last chunk read there)
    static_assert(SLOT_K <= (int)sizeof(g_spare_slot) && SLOT_V <= (int)sizeof(g_spare_slot), "spare slot size");
    for (int i = threadIdx.x; i < kSlotEntries; i += 64 * kWaves) {
      if (i < np) {
        const size_t slot = (size_t)trow[i] * H + kvh;
        sm.kp[i] = (const __attribute__((address_space(1))) uint8_t*)(A.pool_k + slot * SLOT_K);
        sm.vp[i] = (const __attribute__((address_space(1))) uint8_t*)(A.pool_v + slot * SLOT_V);
      } else {
        sm.kp[i] = (const __attribute__((address_space(1))) uint8_t*)g_spare_slot;
        sm.vp[i] = (const __attribute__((address_space(1))) uint8_t*)g_spare_slot;
      }
    }
  }
  // H q of the row tile, stored divided by the weight of each channel's K field
  if (hq_wave) {
    float hq[32];
    const unsigned sgw = sign_word(A.signs, g);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      u32x4 w = row_real ? qraw[v] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] ^= sign_pair_mask_w(sgw, 8 * v, i);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        hq[8 * v + 2 * i] = half_bits_to_float((uint16_t)(w[i] & 0xFFFF));
        hq[8 * v + 2 * i + 1] = half_bits_to_float((uint16_t)(w[i] >> 16));
      }
    }
#pragma unroll
    for (int bit = 1; bit < 32; bit <<= 1)
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        if (i & bit) continue;
        const float lo = hq[i], hi = hq[i | bit];
        hq[i] = lo + hi;
        hq[i | bit] = lo - hi;
      }
    const float s16 = (g & 1) ? -1.f : 1.f, s32 = (g & 2) ? -1.f : 1.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) hq[i] = __builtin_fmaf(hq[i], s16, lane_xor<16>(hq[i]));
#pragma unroll
    for (int i = 0; i < 32; ++i) hq[i] = __builtin_fmaf(hq[i], s32, xor32(hq[i]));
#pragma unroll
    for (int i = 0; i < 32; i += 4) {
      const int c = 32 * g + i;
      f32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = hq[i + e] * (kInvSqrtD / k_field_weight<BK>(c + e));
      *reinterpret_cast<f32x4*>(&sm.hq[16 * rt + n][c]) = o;
    }
  }
  __syncthreads();

  // LDS index of page pj of the sequence; a T = 32 chunk whose second tile
  // was never started reads its first tile's pages instead (every token there
  // is past the end and masked)
  auto page_ix = [&](int pj) { return (pj < npages ? pj : pj - 2) - 4 * c_begin; };
  auto kslot = [&](int pj) { return (const uint8_t*)sm.kp[page_ix(pj)]; };
  auto vslot = [&](int pj) { return (const uint8_t*)sm.vp[page_ix(pj)]; };

  // causal limit of this lane's QK row (padding rows see every token)
  const int vis = row_real ? min(L, L - A.n_q + 1 + my_row / G) : L;
  const float c0 = A.sm_scale_log2;

  float m_run = -INFINITY;   // row n (same in the row's 4 lanes)
  float l_run = 0.f;         // row n, this lane's tokens
  f32x4 acc[8];              // [channel block j]: channel 16 j + n, rows 4 g + i
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // query fold of one tile: qt = hq * alpha_K split hi / lo per k step
  f16x8 qhi[4], qlo[4];
  float cA = 0.f, cB = 0.f;
  // alpha_K of a tile for the lane's channels 16 m + 4 g + j, loaded ahead of its fold
  f32x4 akn[8];
  int akn_page = 0;   // the tile of akn (KCH: its zero offsets are read at the fold)
  auto load_alpha_k = [&](int tile_page) {   // first page (in the sequence) of the tile
    akn_page = tile_page;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int c = 16 * m + 4 * g;
      akn[m] = load_meta4<BK, M16>(kslot(tile_page + c / AL) + ALPHA_K, c % AL);
    }
  };
  auto fold = [&]() {   // the tile whose alpha_K sits in akn
    f32x4 mz[KCH ? 8 : 1];
    if constexpr (KCH) {
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const int c = 16 * m + 4 * g;
        mz[m] = load_meta4<BK, false>(kslot(akn_page + c / AL) + ZP_K, c % AL);
      }
    }
    float x[8][4];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const f32x4 h = *reinterpret_cast<const f32x4*>(&sm.hq[16 * rt + n][16 * m + 4 * g]);
#pragma unroll
      for (int j = 0; j < 4; ++j) x[m][j] = h[j] * akn[m][j];
    }
    float qmax = 0.f;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const float mm = vmax3_abs(x[m][0], x[m][1], vmax3_abs(x[m][2], x[m][3], 0.f));
      qmax = vmax(qmax, mm * k_field_weight<BK>(16 * m));
    }
    qmax = group_max(qmax);   // the row's 4 lanes
    int ex = (int)((__float_as_uint(qmax) >> 23) & 0xFF) - 127;
    ex = min(max(ex, -100), 100);
    const float qscale = __uint_as_float((unsigned)(127 + QE - ex) << 23);
    const float qunscale = __uint_as_float((unsigned)(127 - QE + ex) << 23);
    float qsum = 0.f;
    static_for<0, 4>([&](auto KS_) {
      constexpr int ks = decltype(KS_)::value;
      unsigned hw[4], lw[4];
      static_for<0, 4>([&](auto P_) {
        constexpr int pp = decltype(P_)::value;
        constexpr int m0 = mq_field<BK>(ks, 2 * pp), m1 = mq_field<BK>(ks, 2 * pp + 1);
        constexpr int j0 = mq_off<BK>(ks, 2 * pp), j1 = mq_off<BK>(ks, 2 * pp + 1);
        constexpr float w = k_field_weight<BK>(16 * m0);   // the pair shares its weight
        split_grid(x[m0][j0], x[m1][j1], qscale, qscale, kGrid / w, kGrid / w, hw[pp], lw[pp]);
        if constexpr (KCH) {   // sum_c qt_c M_c over the represented query
          const f16x2 a = __builtin_bit_cast(f16x2, hw[pp]), b = __builtin_bit_cast(f16x2, lw[pp]);
          const float z0 = w * mz[KCH ? m0 : 0][j0], z1 = w * mz[KCH ? m1 : 0][j1];
          qsum = __builtin_fmaf((float)a[0], z0, qsum);
          qsum = __builtin_fmaf((float)b[0], z0, qsum);
          qsum = __builtin_fmaf((float)a[1], z1, qsum);
          qsum = __builtin_fmaf((float)b[1], z1, qsum);
        } else {
          const f16x2 wp{(_Float16)w, (_Float16)w};
          qsum = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, hw[pp]), wp, qsum, false);
          qsum = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, lw[pp]), wp, qsum, false);
        }
      });
      qhi[ks] = as_f16x8(hw[0], hw[1], hw[2], hw[3]);
      qlo[ks] = as_f16x8(lw[0], lw[1], lw[2], lw[3]);
    });
    qsum = group_sum(qsum) * qunscale;
    cA = c0 * kTwo24 * qunscale;   // score = S D cA + O cB
    cB = c0 * qsum;
  };

  // A wave's chunks: c_begin + sub, + nsub, ... (at T = 128 whole tiles: both
  // chunks of a tile, then the tile nsub tiles on)
  constexpr int UNIT = (T == 128) ? 2 : 1;
  auto next_chunk = [&](int c) { return (UNIT == 2 && (c & 1) == 0) ? c + 1 : (c / UNIT + nsub) * UNIT; };

  // Per-chunk operands, loaded one chunk ahead: the code block of the lane's
  // token in each page (K), the quad words of its runs (V), and the scales and
  // offsets of token `lane` (spread to the lanes' tokens through LDS)
  struct Ops {
    u32x4 kb[4][BK == 8 ? 2 : 1];
    unsigned vw[4][4][BV == 8 ? 2 : 1];   // [run group jr][page][word]
    float sk, ok, sv, ov;
  };
  auto load_k_ops = [&](Ops& o, int c) {
    const int pg0 = 4 * c;
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      const uint8_t* sl = kslot(pg0 + tb);
      if constexpr (BK == 8) {
        o.kb[tb][0] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(sl + 32 * (16 * g + n)));
        o.kb[tb][1] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(sl + 32 * (16 * g + n) + 16));
      } else if constexpr (BK == 4) {
        o.kb[tb][0] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(sl + 16 * (16 * g + n)));
      } else {
        const u32x2 w = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(sl + 8 * (16 * g + n)));
        o.kb[tb][0] = u32x4{w[0], w[1], 0u, 0u};
      }
    }
  };
  auto load_v_ops = [&](Ops& o, int c) {
    const int pg0 = 4 * c;
#pragma unroll
    for (int jr = 0; jr < 4; ++jr)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint8_t* vs = vslot(pg0 + q);
        const int run = 16 * jr + n;
        if constexpr (BV == 8) {
          const u32x2 w = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(vs + 32 * run + 8 * g));
          o.vw[jr][q][0] = w[0];
          o.vw[jr][q][1] = w[1];
        } else if constexpr (BV == 4) {
          o.vw[jr][q][0] = __builtin_nontemporal_load(reinterpret_cast<const unsigned*>(vs + 16 * run + 4 * g));
        } else {
          o.vw[jr][q][0] = __builtin_nontemporal_load(reinterpret_cast<const unsigned*>(vs + 8 * run + 4 * (g >> 1)));
        }
      }
  };
  auto load_meta_ops = [&](Ops& o, int c) {
    const int pg0 = 4 * c;
    const uint8_t* ks = kslot(pg0 + (lane >> 4));
    const uint8_t* vs = vslot(pg0 + (lane >> 4));
    o.sk = load_meta<M16>(ks + CODE_K, lane & 15);
    o.ok = KCH ? o.sk : load_meta<M16>(ks + OFF_K, lane & 15);   // KCH: beta for both
    o.sv = load_meta<M16>(vs + CODE_V, lane & 15);
    o.ov = load_meta<M16>(vs + OFF_V, lane & 15);
  };

  // one chunk; the operands of the next one (cn < c_end) are loaded into o
  // as soon as the current ones are used
  auto process = [&](Ops& o, int chunk, int cn) {
    const int pg0 = 4 * chunk;
    const bool more = cn < c_end;
    // loads for the next chunk go out unconditionally (past the last they read
    // the spare slot) so that the loop keeps no in-flight register to copy at
    // its end
    const int spare = c_begin + kMaxChunksPerPart;
    const int ld = more ? cn : spare;
    // P = p S_V, scaled by 2^k per chunk so that it stays below 2^(PE+1)
    const float smax = wave_max(vmax(o.sv, 0.f));
    int pe = (int)((__float_as_uint(smax) >> 23) & 0xFF) - 127;
    pe = min(max(pe, -100), 100);
    const float pk = (float)(PE - pe);
    const float pinv = __uint_as_float((unsigned)(127 - PE + pe) << 23);   // 2^-k
    // per token (lane = token of the chunk): the V scale the probabilities are
    // multiplied by (a zero-range token, S = 0 and codes 0, takes 2^pe <= max S_V
    // in place of S: its P then carries p to the offset term while its codes
    // contribute nothing; tokens 2, 3 of a quad divided by kTok) and O over it,
    // nearest (reciprocal refined by one Newton step)
    float swt = o.sv > 0.f ? o.sv : __uint_as_float((unsigned)(127 + pe) << 23);
    if ((lane & 3) >= 2) swt *= (1.f / kTok);
    const float rct = __builtin_amdgcn_rcpf(swt);
    const float z0t = o.ov * rct;
    const float zrt = __builtin_fmaf(__builtin_fmaf(-swt, z0t, o.ov), rct, z0t);
    float* meta = sm.meta[wave];   // [4][64]: S_K, O_K, sw, O / sw by token of the chunk
    meta[lane] = o.sk;
    meta[64 + lane] = o.ok;
    meta[128 + lane] = swt;
    meta[192 + lane] = zrt;
    asm volatile("" ::: "memory");   // the reads below see this wave's writes (LDS keeps order)
    load_meta_ops(o, ld);
    // alpha_V of the lane's channels 16 j + n for the chunk's tile(s), needed after the softmax
    float av[T == 32 ? 2 : 1][8];
#pragma unroll
    for (int tt = 0; tt < (T == 32 ? 2 : 1); ++tt) {
      const int tp = (T == 32) ? pg0 + 2 * tt : (T == 64 ? pg0 : 4 * (chunk & ~1));
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int ch = 16 * j + n;
        av[tt][j] = load_meta<M16>(vslot(tp + ch / AL) + ALPHA_V, ch % AL);
      }
    }

    // ---------------------------------------------- QK: per page tb of the chunk
    if (T == 64 || (T == 128 && (chunk & 1) == 0)) {
      fold();
      const int cn = (T == 128) ? next_chunk(next_chunk(chunk)) : next_chunk(chunk);   // the next tile's chunk
      load_alpha_k(4 * (cn < c_end ? cn : spare));
    }
    float s[4][4];   // [page][i]: token 64 chunk + 16 tb + 4 g + i, row n
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      if (T == 32 && (tb & 1) == 0) {   // a tile per two pages
        fold();
        const int cn = next_chunk(chunk);
        if (tb == 0) load_alpha_k(pg0 + 2);
        else load_alpha_k(4 * (cn < c_end ? cn : spare));
      }
      const f32x4 sk = *reinterpret_cast<const f32x4*>(&meta[16 * tb + 4 * g]);
      const f32x4 ok = *reinterpret_cast<const f32x4*>(&meta[64 + 16 * tb + 4 * g]);
      // the lo products go on top of the finished (exact) hi sum: one rounding per add
      f32x4 d{0.f, 0.f, 0.f, 0.f};
      f16x8 a[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        a[ks] = mq_k_operand<BK>(o.kb[tb], ks);
        d = mfma16(a[ks], qhi[ks], d);
      }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) d = mfma16(a[ks], qlo[ks], d);
#pragma unroll
      for (int i = 0; i < 4; ++i) s[tb][i] = __builtin_fmaf(cA * sk[i], d[i], cB * ok[i]);
    }
    load_k_ops(o, ld);
    // causal and length mask, only where some row's limit falls inside the chunk
    if (__builtin_amdgcn_ballot_w64(vis < kChunk * (chunk + 1)) != 0) {
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (kChunk * chunk + 16 * tb + 4 * g + i >= vis) s[tb][i] = -INFINITY;
    }

    // ---------------------------------------------- online softmax (base 2), row n
    float cm = s[0][0];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int i = 0; i < 4; ++i) cm = vmax(cm, s[tb][i]);
    cm = group_max(cm);
    const float m_new = vmax(m_run, cm);
    // a row that has seen no visible token yet keeps m = -inf (p = 0)
    const float corr = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
    const float mb = (m_new == -INFINITY) ? 0.f : m_new;
    m_run = m_new;
    l_run *= corr;
    if (__builtin_amdgcn_ballot_w64(corr != 1.f) != 0) {   // rescale the PV rows 4 g + i
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float ci = __shfl(corr, 4 * g + i);
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j][i] *= ci;
      }
    }
    float p[4][4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[tb][i] = __builtin_amdgcn_exp2f(s[tb][i] - (mb - pk));
        l_run = __builtin_fmaf(p[tb][i], pinv, l_run);
      }

    // ---------------------------------------------- PV operands per pair of pages (32 tokens)
    f16x8 pah[2], pal[2];
    float po[2] = {0.f, 0.f};   // sum_t P_t O_t / sw_t per page pair (row n, this lane's tokens)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      unsigned ph[4], pl[4];
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2) {
        const int tb = 2 * kb + q2;
        const f32x4 sw = *reinterpret_cast<const f32x4*>(&meta[128 + 16 * tb + 4 * g]);
        const f32x4 zr = *reinterpret_cast<const f32x4*>(&meta[192 + 16 * tb + 4 * g]);
        split_grid(p[tb][0], p[tb][1], sw[0], sw[1], kGrid, kGrid, ph[2 * q2], pl[2 * q2]);
        split_grid(p[tb][2], p[tb][3], sw[2], sw[3], kGrid / kTok, kGrid / kTok, ph[2 * q2 + 1], pl[2 * q2 + 1]);
        // offset term through the represented P: p_t O_t = P_t (O_t / sw_t)
        const f16x2 a = __builtin_bit_cast(f16x2, ph[2 * q2]), b = __builtin_bit_cast(f16x2, pl[2 * q2]);
        const f16x2 c = __builtin_bit_cast(f16x2, ph[2 * q2 + 1]), e = __builtin_bit_cast(f16x2, pl[2 * q2 + 1]);
        float& q = po[kb];
        q = __builtin_fmaf((float)a[0], zr[0], q);
        q = __builtin_fmaf((float)b[0], zr[0], q);
        q = __builtin_fmaf((float)a[1], zr[1], q);
        q = __builtin_fmaf((float)b[1], zr[1], q);
        q = __builtin_fmaf((float)c[0], zr[2], q);
        q = __builtin_fmaf((float)e[0], zr[2], q);
        q = __builtin_fmaf((float)c[1], zr[3], q);
        q = __builtin_fmaf((float)e[1], zr[3], q);
      }
      pah[kb] = as_f16x8(ph[0], ph[1], ph[2], ph[3]);
      pal[kb] = as_f16x8(pl[0], pl[1], pl[2], pl[3]);
    }
    // the per-row offset terms of the fold segments (a page pair at T = 32,
    // the chunk otherwise), moved to the PV rows 4 g + i
    constexpr int NSEG = (T == 32) ? 2 : 1;
    float so[NSEG][4];
#pragma unroll
    for (int sg = 0; sg < NSEG; ++sg) {
      const float pos = group_sum(NSEG == 2 ? po[sg] : po[0] + po[1]) * pinv;   // row n
#pragma unroll
      for (int i = 0; i < 4; ++i) so[sg][i] = __shfl(pos, 4 * g + i);
    }

    // ---------------------------------------------- PV: channels 16 jr + n and 64 + 16 jr + n
#pragma unroll
    for (int jr = 0; jr < 4; ++jr) {
#pragma unroll
      for (int sg = 0; sg < NSEG; ++sg) {
        constexpr int KB0 = 0, NKB = (NSEG == 2) ? 1 : 2;   // page pairs of the segment
        f32x4 vh[2];   // [channel half]: the hi chain (exact), then the lo products on top
        f16x8 bv[2][2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          vh[h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = KB0; kk < NKB; ++kk) {
            const int kb = (NSEG == 2) ? sg : kk;
            unsigned b[4];
#pragma unroll
            for (int q2 = 0; q2 < 2; ++q2) {
              unsigned x = o.vw[jr][2 * kb + q2][0];
              if (BV == 2 && (g & 1)) x >>= 8;   // odd quads sit in bits 8..15 of each half
              mq_v_fields<BV>(x, BV == 8 ? o.vw[jr][2 * kb + q2][BV == 8 ? 1 : 0] : 0u, h, b[2 * q2], b[2 * q2 + 1]);
            }
            bv[h][kk] = as_f16x8(b[0], b[1], b[2], b[3]);
            vh[h] = mfma16(pah[kb], bv[h][kk], vh[h]);
          }
        }
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int kk = KB0; kk < NKB; ++kk) vh[h] = mfma16(pal[(NSEG == 2) ? sg : kk], bv[h][kk], vh[h]);
        // acc += alpha_V (sum_t p_t S_t k_t + sum_t p_t O_t) over the segment
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int j = jr + 4 * h;
          const float cf = kTwo24 * pinv * ((BV == 2 && h == 1) ? (1.f / 16.f) : 1.f);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[j][i] = __builtin_fmaf(av[sg][j], __builtin_fmaf(vh[h][i], cf, so[sg][i]), acc[j][i]);
        }
      }
    }
    load_v_ops(o, ld);
  };

  if (active) {
    int c = c_begin + sub * UNIT;
    Ops o;
    if (c < c_end) {
      load_alpha_k(4 * (T == 128 ? (c & ~1) : c));
      load_k_ops(o, c);
      load_v_ops(o, c);
      load_meta_ops(o, c);
    }
    while (c < c_end) {
      const int cn = next_chunk(c);
      process(o, c, cn);
      c = cn;
    }
  }

  // ------------------------------------------------ merge the waves of each row tile, write partials
  l_run = group_sum(l_run);
  __syncthreads();   // every wave is done with the query rows
  if (active) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.merge.acc[wave][4 * g + i][16 * j + n] = acc[j][i];
    if (g == 0) {
      sm.merge.m[wave][n] = m_run;
      sm.merge.l[wave][n] = l_run;
    }
  }
  __syncthreads();
  // thread -> (row of the block, 4 channels)
  for (int it = threadIdx.x; it < nrows * 32; it += 64 * kWaves) {
    const int r = it >> 5, c = 4 * (it & 31);
    const int t = r >> 4, rr = r & 15;   // row tile, row in it; waves t, t + nrt, ...
    float M = -INFINITY;
    for (int s2 = 0; s2 < nsub; ++s2) M = fmaxf(M, sm.merge.m[t + s2 * nrt][rr]);
    float lsum = 0.f;
    f32x4 x{0.f, 0.f, 0.f, 0.f};
    for (int s2 = 0; s2 < nsub; ++s2) {
      const int w = t + s2 * nrt;
      const float mw = sm.merge.m[w][rr];
      const float wt = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw - M);
      lsum = __builtin_fmaf(wt, sm.merge.l[w][rr], lsum);
      const f32x4 y = *reinterpret_cast<const f32x4*>(&sm.merge.acc[w][rr][c]);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = __builtin_fmaf(wt, y[e], x[e]);
    }
    const int rg = r0 + r;
    const size_t pidx = (((size_t)seq * A.n_q + rg / G) * A.q_heads + kvh * G + rg % G) * A.max_parts + part;
    *reinterpret_cast<f32x4*>(A.ws_acc + pidx * kHeadDim + c) = x;
    if (c == 0) {
      A.ws_ml[2 * pidx] = M;
      A.ws_ml[2 * pidx + 1] = lsum;
    }
  }
}

// Multi-query attention with at least 16 rows ((query, head) pairs) per
// sequence and kv head: workgroups of up to 64 rows, then the partition merge.
template <int FMT>
hipError_t launch_mq_dense_fmt(const DecodeArgs& a, int tile, int bits_k, int bits_v, hipStream_t s) {
  return by_tile(tile, [&](auto T) {
    return by_format<FMT>(bits_k, bits_v, [&](auto BK, auto BV) {
      constexpr bool M16 = FMT == kFmtM16, KCH = FMT == kFmtKch;
      const int rows = a.n_q * a.group;
      dim3 grid(a.kv_heads * ((rows + kMqBlockRows - 1) / kMqBlockRows) * a.num_seqs, a.max_parts);
      hipLaunchKernelGGL((mq_dense_kernel<T(), BK(), BV(), M16, KCH>), grid, dim3(64 * kWaves), 0, s, a);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      return launch_combine(a, 64, true, s);
    });
  });
}

}  // namespace
}  // namespace kvq
