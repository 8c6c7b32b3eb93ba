// HIP kernels for windowed-RoPE attention on gfx950 (CDNA4).
//
// Method (source page "ATFlash: RoPE-Frequenzen kuerzen Attention-Arbeit um
// bis zu 57 Prozent", sudo-ai.de, section "Was ATFlash anders macht"): rotary
// pair p keeps its share q'_p k'_p + q'_{p+P} k'_{p+P} of score(i,j) only while
// the distance i - j is at most W_p, a window proportional to the pair's
// wavelength; the slowest pair is never cut.  Section "Die Zahlen - und ihre
// Grenze": the online-softmax recurrence stays as it is.
//
// Windows are non-decreasing in p, so at distance D the kept pairs are the
// suffix [p*(D), P) with p*(D) = #{p : W_p < D}.  Everything below is built on
// that fact: in the pair-interleaved key layout the kept dims of a tile are
// one contiguous K-range of the MFMA contraction.

#include "atf_internal.h"

#include <math.h>

#include <algorithm>
#include <type_traits>
#include <mutex>

namespace atf {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
// native vector types (HIP's u32x4/u32x2 are structs and defeat register promotion)
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr double kTwoPiHi = 6.283185307179586;       // double nearest to 2*pi
constexpr double kTwoPiLo = 2.4492935982947064e-16;  // 2*pi - kTwoPiHi
constexpr double kInvTwoPi = 0.15915494309189535;

// cos and sin of pos * theta.  The angle is formed and reduced to [-pi, pi]
// in fp64 (a two-constant 2*pi), so positions up to 2^31 keep ~1e-7 rad
// accuracy; only the final sincos runs in fp32.
__device__ inline void rope_cos_sin(long long pos, double theta, float &c, float &s) {
    const double a = (double)pos * theta;
    const double k = rint(a * kInvTwoPi);
    double r = fma(-k, kTwoPiHi, a);
    r = fma(-k, kTwoPiLo, r);
    sincosf((float)r, &s, &c);
}

__device__ inline float bf_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ inline float bf_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats to a packed bf16 pair, round to nearest even.
__device__ inline unsigned pack_bf(float lo, float hi) {
    bf16x2_t v;
    v[0] = (__bf16)lo;
    v[1] = (__bf16)hi;
    return __builtin_bit_cast(unsigned, v);
}

__device__ inline float dot2_bf(unsigned a, unsigned b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Rotary pairs off .. off+3 of a bf16 row as two 8-byte pieces.  NeoX
// half-split layout (pair p = dims p and p + P): lo holds the pairs' first
// elements, hi their second.  GPT-J interleaved layout (pair p = dims 2p and
// 2p + 1): lo holds pairs off, off+1 and hi pairs off+2, off+3, each pair one
// 32-bit word (first element in the low half).
__device__ inline void load_pair_pieces(const unsigned short *row, int off, int P, bool gptj, u32x2 &lo, u32x2 &hi) {
    if (gptj) {
        lo = *(const u32x2 *)(row + 2 * off);
        hi = *(const u32x2 *)(row + 2 * off + 4);
    } else {
        lo = *(const u32x2 *)(row + off);
        hi = *(const u32x2 *)(row + P + off);
    }
}
// The window table spread over a wave: lane l holds W_l and, for d = 256,
// W_{l+64} (kWindowInf past the table).  W_p grows with p, so the cut prefix at
// distance x, #{p : W_p < x}, is one ballot count per half.
template <int P>
struct WaveWin {
    int lo, hi;
};
template <int P>
__device__ inline WaveWin<P> load_windows(const int *W) {
    const int lane = threadIdx.x & 63;
    WaveWin<P> w;
    w.lo = (lane < P) ? W[lane] : kWindowInf;
    w.hi = (P > 64 && lane + 64 < P) ? W[lane + 64] : kWindowInf;
    return w;
}
template <int P>
__device__ inline int cut_below(const WaveWin<P> &w, int x) {
    int n = __builtin_popcountll(__ballot(w.lo < x));
    if constexpr (P > 64) n += __builtin_popcountll(__ballot(w.hi < x));
    return n;
}
// W_p for a wave-uniform p
template <int P>
__device__ inline int window_at(const WaveWin<P> &w, int p) {
    const int a = __builtin_amdgcn_readlane(w.lo, p & 63);
    if constexpr (P > 64) return (p < 64) ? a : __builtin_amdgcn_readlane(w.hi, p & 63);
    return a;
}

// First (x) and second (y) element of pair off + w (w = 0..3) from the pieces.
__device__ inline void pair_xy(u32x2 lo, u32x2 hi, int w, bool gptj, float &x, float &y) {
    if (gptj) {
        const unsigned wd = (w == 0) ? lo.x : (w == 1) ? lo.y : (w == 2) ? hi.x : hi.y;
        x = __uint_as_float(wd << 16);
        y = __uint_as_float(wd & 0xffff0000u);
    } else {
        const unsigned lw = (w < 2) ? lo.x : lo.y, hw = (w < 2) ? hi.x : hi.y;
        x = (w & 1) ? __uint_as_float(lw & 0xffff0000u) : __uint_as_float(lw << 16);
        y = (w & 1) ? __uint_as_float(hw & 0xffff0000u) : __uint_as_float(hw << 16);
    }
}

__device__ inline unsigned long long wave_sum_u64(unsigned long long v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// LDS swizzles.  A 64-lane ds_read_b128 is served 8 or 16 lanes per pass;
// these make the 8 and the 16 rows read in one pass land in distinct bank
// groups for 128-byte rows (swz8) and 256-byte rows (swz16).
__device__ inline int swz8(int row) { return ((row >> 1) ^ ((row & 1) << 2)) & 7; }
__device__ inline int swz16(int row) { return row & 15; }
template <int CH>
__device__ inline int kswz(int row) { return (CH >= 16) ? swz16(row) : swz8(row); }
template <int CH>
constexpr int kswz_rows() { return (CH >= 16) ? 16 : 8; }  // period of kswz in rows

// ============================================================================
// Preparation pass (bf16): rotate every key once, store it pair-interleaved
// (dims (p, p+P) side by side as one 32-bit word), and store the values
// transposed per 64-key tile, keys permuted inside each group of 16 so that
// the attention kernel's MFMA operand for P.V is one 16-byte LDS read.
// Keys [k_begin, k_end) come from source rows 0 .. k_end - k_begin - 1; keys
// past k_end are cleared, keys before k_begin (the first tile of an append
// that does not start on a tile) are kept.
// grid (number of 64-key tiles from tile0, B*Hkv, d/32: 16 pairs each), block 256.
// ============================================================================

// Key held at position `pos` (0..15) of a 16-key group of a value tile.
__device__ inline int vt_key_of_pos(int pos) {
    const int h = pos >> 3, e = pos & 7;
    return ((e >> 2) << 3) + (h << 2) + (e & 3);
}

template <int D>
__global__ __launch_bounds__(256) void prep_bf16_kernel(PrepArgs a) {
    constexpr int P = D / 2;
    constexpr int PPT = 4;  // pairs per thread: block z rotates pairs 16 z .. 16 z + 15 of the tile's 64 keys
    const int tile = a.tile0 + blockIdx.x, bh = blockIdx.y, t = threadIdx.x, z = blockIdx.z;
    // source rows: key j is row j - k_begin
    const unsigned short *k = (const unsigned short *)a.k + (long long)bh * a.src_rows * D;
    const unsigned short *v = (const unsigned short *)a.v + (long long)bh * a.src_rows * D;
    unsigned *kr = (unsigned *)a.krot + (long long)bh * a.S_pad * P;
    unsigned short *vt = (unsigned short *)a.vt + ((long long)bh * (a.S_pad / kKeyTile) + tile) * (D * kKeyTile);

    if (a.counter && blockIdx.x == 0 && bh == 0 && z == 0 && t == 0) *a.counter = 0ull;

    {  // keys
        const int row = t >> 2, p0 = 16 * z + (t & 3) * PPT;
        const int j = tile * kKeyTile + row;
        union { u32x4 v[PPT / 4]; unsigned w[PPT]; } res;
        if (j >= a.k_begin && j < a.k_end) {
            const unsigned short *src = k + (long long)(j - a.k_begin) * D;
            const long long pos = a.pos0 + j;
            u32x2 lo[PPT / 4], hi[PPT / 4];
#pragma unroll
            for (int g = 0; g < PPT / 4; ++g) load_pair_pieces(src, p0 + 4 * g, P, a.gptj != 0, lo[g], hi[g]);
#pragma unroll
            for (int u = 0; u < PPT; ++u) {
                float c, s, x, y;
                rope_cos_sin(pos, a.theta[p0 + u], c, s);
                pair_xy(lo[u / 4], hi[u / 4], u % 4, a.gptj != 0, x, y);
                res.w[u] = pack_bf(x * c - y * s, y * c + x * s);
            }
        } else {
#pragma unroll
            for (int u = 0; u < PPT; ++u) res.w[u] = 0u;
        }
        u32x4 *dst = (u32x4 *)(kr + (long long)j * P + p0);
        if (j >= a.k_begin) {
#pragma unroll
            for (int u = 0; u < PPT / 4; ++u) dst[u] = res.v[u];
        }
    }

    if (z != 0) return;  // the values of the tile: block z = 0
    {  // values: tile [64][D] -> LDS -> [D][64] with the in-group key permutation
        constexpr int LD = D + 8;  // padded LDS row (ushort)
        __shared__ unsigned short vs[kKeyTile * LD];
        constexpr int CHR = D / 8;  // 16-byte chunks per row
#pragma unroll
        for (int n = 0; n < (kKeyTile * CHR) / 256; ++n) {
            const int g = t + 256 * n;
            const int row = g / CHR, ch = g % CHR;
            const int j = tile * kKeyTile + row;
            u32x4 val = (u32x4){0u, 0u, 0u, 0u};
            if (j >= a.k_begin && j < a.k_end) val = *(const u32x4 *)(v + (long long)(j - a.k_begin) * D + ch * 8);
            *(u32x4 *)(vs + row * LD + ch * 8) = val;
        }
        __syncthreads();
        const int keep = a.k_begin - tile * kKeyTile;  // keys of this tile already in place
#pragma unroll
        for (int n = 0; n < (D * 8) / 256; ++n) {
            const int g = t + 256 * n;
            const int dim = g >> 3, pc = g & 7;
            union { u32x4 v; unsigned short s[8]; } o, old;
            old.v = (u32x4){0u, 0u, 0u, 0u};
            if (keep > 0) old.v = *(const u32x4 *)(vt + dim * kKeyTile + pc * 8);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int pos = pc * 8 + e;
                const int key = (pos & ~15) + vt_key_of_pos(pos & 15);
                o.s[e] = key < keep ? old.s[e] : vs[key * LD + dim];
            }
            *(u32x4 *)(vt + dim * kKeyTile + pc * 8) = o.v;
        }
    }
}

// ============================================================================
// Prefill attention, bf16 in / fp32 accumulate, MFMA 32x32x16.
//
// d <= 128 (d = 256 runs on prefill16_bf16_kernel below).
// Workgroup = 8 waves (two per SIMD) = 256 queries of one (b, h); wave w owns
// 32 queries.  Key tiles of 128 keys stream global -> LDS with direct LDS loads
// (buffer_load_dwordx4 ... lds: no staging registers, the tile base advances
// in scalar registers), double-buffered, one barrier per tile.  Per 32-key
// block each wave computes a 32x32 score block S^T = K' Q'^T (keys on MFMA
// rows, queries on columns: a lane holds 16 keys of one query, its partner
// lane^32 the other 16, so softmax row statistics need one lane swap), then
// O^T += V^T P^T.  Blocks go in pairs, chain0 | chain1 + probs0 | PV0 +
// probs1 | PV1, so the exponentials sit beside MFMA runs.  Tiles where every
// key precedes every query of the wave (non-causal: or follows every query)
// and no window falls inside the tile's distance range take a fast path with
// one pair cut for all their blocks.
//
// Windows per 32x32 block: distances span [dmin, dmax]; pairs below
// p_lo = p*(dmin) are dropped everywhere in the block, pairs from
// p_full = p*(dmax) on are kept everywhere.  The MFMA K-loop runs only over
// the 16-dim steps holding pairs >= p_full; pairs below p_full inside the
// first step are zeroed in the key operand (exact: the block is uniform
// there).  The loop is one of NSTEP straight-line variants chosen once per
// block, so its LDS reads can be hoisted.  Each boundary pair p in
// [p_lo, p_full) gets its own MFMA with a key operand holding only pair p,
// added element by element where the distance is within W_p.  Dropped terms
// are counted exactly.
//
// Scores come out in log2 units and already shifted by the softmax reference:
// q' is pre-scaled by log2(e)/sqrt(d), and each score chain starts with a
// rank-1 MFMA that puts -m_ref in every element, so a probability is 2^score.
// ============================================================================

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

__device__ inline float quad_max(float x) {  // max over lanes t, t+16, t+32, t+48
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b2[0]), __uint_as_float(b2[1]));
}
__device__ inline float quad_sum(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b2[0]) + __uint_as_float(b2[1]);
}

__device__ inline float partner_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float partner_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

typedef __attribute__((address_space(3))) void lds_void_t;

// 16 bytes per lane, global -> LDS, no registers: lane l of the wave writes
// LDS bytes [dst + 16 l, dst + 16 l + 16); dst must be wave-uniform.
__device__ inline void lds_dma16(const void *src, void *dst) {
    __builtin_amdgcn_global_load_lds(src, (lds_void_t *)dst, 16, 0, 0);
}

// Buffer resource for `bytes` bytes at a wave-uniform base (raw, unswizzled);
// reads at offsets >= bytes return zero instead of touching memory.
__device__ inline __amdgpu_buffer_rsrc_t raw_rsrc(const void *base, unsigned bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// Same as lds_dma16, addressed as buffer base (SGPRs) + per-lane byte offset,
// so advancing the base costs no vector instructions.
__device__ inline void lds_dma16_buf(__amdgpu_buffer_rsrc_t r, unsigned voff, int soff, void *dst) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)dst, 16, (int)voff, soff, 0, 0);
}

// 16 bytes at buffer offset voff (zeros, without a memory access, past the end).
__device__ inline u32x4 raw_load16(__amdgpu_buffer_rsrc_t r, unsigned voff) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 0));
}

// One block's main score chain starting at K-step S0 (compile time).
// kaddr(s) = kbase + ((32 s) ^ ky): the swizzled byte address of this lane's
// 16 key dims of step s.
template <int NSTEP, int S0>
__device__ inline f32x16_t qk_chain(const unsigned char *lds, unsigned kbase, unsigned ky,
                                    const bf16x8_t *qf, int zero_below, s16x4_t ones_a, s16x4_t negm_b) {
    u32x4 kw = *(const u32x4 *)(lds + kbase + ((32u * S0) ^ ky));
    // words (pairs) of the first step below p_full are dropped or boundary
    kw.x = (0 < zero_below) ? 0u : kw.x;
    kw.y = (1 < zero_below) ? 0u : kw.y;
    kw.z = (2 < zero_below) ? 0u : kw.z;
    kw.w = (3 < zero_below) ? 0u : kw.w;
    const f32x16_t zero16 = {};
    // -m_ref of each query column in every element: one rank-1 product (a column
    // of ones times the row of -m_ref, on the K = 8 MFMA whose operands take
    // two registers each), so the scores leave the chain already shifted by
    // the softmax reference
    f32x16_t acc = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(ones_a, negm_b, zero16, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kw), qf[S0], acc, 0, 0, 0);
#pragma unroll
    for (int s = S0 + 1; s < NSTEP; ++s) {
        const u32x4 k2 = *(const u32x4 *)(lds + kbase + ((32u * s) ^ ky));
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, k2), qf[s], acc, 0, 0, 0);
    }
    return acc;
}

template <int NSTEP>
__device__ inline f32x16_t qk_main(int s_first, const unsigned char *lds, unsigned kbase, unsigned ky,
                                   const bf16x8_t *qf, int zero_below, s16x4_t ones_a, s16x4_t negm_b) {
#define ATF_CHAIN(s0_) qk_chain<NSTEP, s0_>(lds, kbase, ky, qf, zero_below, ones_a, negm_b)
    // s_first < NSTEP (the slowest pair is never cut); the last step is also
    // the fall-through
#define ATF_C(i) \
    case i:      \
        if constexpr ((i) < NSTEP - 1) return ATF_CHAIN((i) < NSTEP - 1 ? (i) : 0); else break;
    switch (s_first) { ATF_C(0) ATF_C(1) ATF_C(2) ATF_C(3) ATF_C(4) ATF_C(5) ATF_C(6) ATF_C(7)
                       ATF_C(8) ATF_C(9) ATF_C(10) ATF_C(11) ATF_C(12) ATF_C(13) ATF_C(14) default: break; }
#undef ATF_C
    return ATF_CHAIN(NSTEP - 1);
#undef ATF_CHAIN
}

// Smallest bf16 value >= x (finite x): the softmax reference is kept exactly
// representable in bf16 so the score MFMA can subtract it.
__device__ inline float bf16_ceil(float x) {
    const unsigned u = __float_as_uint(x);
    return __uint_as_float((u & 0x80000000u) ? (u & 0xffff0000u) : ((u + 0xffffu) & 0xffff0000u));
}

// Number of a lane's 16 key slots c_r = 8(r/4) + r%4 (r = 0..15) with c_r < x.
__device__ inline int keys_below(int x) {
    int n = 0;
#pragma unroll
    for (int g = 0; g < 4; ++g) n += min(max(x - 8 * g, 0), 4);
    return n;
}

// Probabilities 2^s of one 32x32 score block (a lane's 16 keys) as 8 bf16
// pairs, and their sum, taken in fp32 before the rounding.  The sum is a tree
// of fp32 adds, which issue beside the P.V MFMAs; v_dot2 over the rounded
// pairs (the sum exactly as the MFMA sees it) does not overlap MFMAs on
// gfx950 and cost about 1% of the kernel.
__device__ __attribute__((always_inline)) inline void block_probs(const f32x16_t &s, unsigned (&pw)[8],
                                                                   float &lsum) {
    float t[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const float e0 = fast_exp2(s[2 * u]), e1 = fast_exp2(s[2 * u + 1]);
        pw[u] = pack_bf(e0, e1);
        t[u] = e0 + e1;
    }
    lsum = ((t[0] + t[1]) + (t[2] + t[3])) + ((t[4] + t[5]) + (t[6] + t[7]));
}

// O^T += V^T P^T for one 32-key block of the tile in LDS (lt): two K-steps
// of 16 keys, NDB output blocks of 32 dims.
template <int NDB>
__device__ __attribute__((always_inline)) inline void block_pv(f32x16_t (&o)[NDB], const unsigned char *lt,
                                                                unsigned vbase_lane, unsigned vz, int kb,
                                                                const unsigned (&pw)[8]) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const unsigned vaddr = vbase_lane + ((32u * (2 * kb + t)) ^ vz);
        const bf16x8_t pop = __builtin_bit_cast(bf16x8_t, (u32x4){pw[4 * t], pw[4 * t + 1], pw[4 * t + 2], pw[4 * t + 3]});
#pragma unroll
        for (int db = 0; db < NDB; ++db)
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8_t, *(const u32x4 *)(lt + vaddr + db * (32 * 128))), pop, o[db], 0, 0, 0);
    }
}

// Second block's score chain and the first block's probabilities, written as
// one straight-line sequence so the exponentials issue between the MFMAs.
template <int NSTEP, int S0>
__device__ __attribute__((always_inline)) inline f32x16_t qk_chain_probs(
    const unsigned char *lds, unsigned kbase, unsigned ky, const bf16x8_t *qf, int zero_below, s16x4_t ones_a,
    s16x4_t negm_b, const f32x16_t &sp, unsigned (&pw)[8], float &lsum) {
    const f32x16_t acc = qk_chain<NSTEP, S0>(lds, kbase, ky, qf, zero_below, ones_a, negm_b);
    block_probs(sp, pw, lsum);
    return acc;
}

template <int NSTEP>
__device__ inline f32x16_t qk_main_probs(int s_first, const unsigned char *lds, unsigned kbase, unsigned ky,
                                         const bf16x8_t *qf, int zero_below, s16x4_t ones_a, s16x4_t negm_b,
                                         const f32x16_t &sp, unsigned (&pw)[8], float &lsum) {
#define ATF_CHAIN(s0_) qk_chain_probs<NSTEP, s0_>(lds, kbase, ky, qf, zero_below, ones_a, negm_b, sp, pw, lsum)
    // s_first < NSTEP (the slowest pair is never cut); the last step is also
    // the fall-through
#define ATF_C(i) \
    case i:      \
        if constexpr ((i) < NSTEP - 1) return ATF_CHAIN((i) < NSTEP - 1 ? (i) : 0); else break;
    switch (s_first) { ATF_C(0) ATF_C(1) ATF_C(2) ATF_C(3) ATF_C(4) ATF_C(5) ATF_C(6) ATF_C(7)
                       ATF_C(8) ATF_C(9) ATF_C(10) ATF_C(11) ATF_C(12) ATF_C(13) ATF_C(14) default: break; }
#undef ATF_C
    return ATF_CHAIN(NSTEP - 1);
#undef ATF_CHAIN
}

// Both score chains of a pair of blocks that share one pair cut (first kept
// K-step S0) and the first block's probabilities: one straight-line run per
// S0.  The exponentials depend on the first chain and the run ends with the
// second, so they stay inside the run, beside the second chain's MFMAs.
template <int NSTEP, int S0>
__device__ __attribute__((always_inline)) inline void qk_pair_chain(
    const unsigned char *lds, unsigned kb0, unsigned kb1, unsigned ky, const bf16x8_t *qf, int zero_below,
    s16x4_t ones_a, s16x4_t negm_b, f32x16_t &s0, f32x16_t &s1, unsigned (&pw)[8], float &lsum) {
    s0 = qk_chain<NSTEP, S0>(lds, kb0, ky, qf, zero_below, ones_a, negm_b);
    block_probs(s0, pw, lsum);
    s1 = qk_chain<NSTEP, S0>(lds, kb1, ky, qf, zero_below, ones_a, negm_b);
}

template <int NSTEP>
__device__ inline void qk_pair(int s_first, const unsigned char *lds, unsigned kb0, unsigned kb1, unsigned ky,
                               const bf16x8_t *qf, int zero_below, s16x4_t ones_a, s16x4_t negm_b, f32x16_t &s0,
                               f32x16_t &s1, unsigned (&pw)[8], float &lsum) {
#define ATF_PAIR(s0_) \
    qk_pair_chain<NSTEP, s0_>(lds, kb0, kb1, ky, qf, zero_below, ones_a, negm_b, s0, s1, pw, lsum)
    // s_first < NSTEP (the slowest pair is never cut); the last step is also
    // the fall-through
#define ATF_C(i)                                                        \
    case i:                                                             \
        if constexpr ((i) < NSTEP - 1) { ATF_PAIR((i) < NSTEP - 1 ? (i) : 0); return; } else break;
    switch (s_first) { ATF_C(0) ATF_C(1) ATF_C(2) ATF_C(3) ATF_C(4) ATF_C(5) ATF_C(6) ATF_C(7)
                       ATF_C(8) ATF_C(9) ATF_C(10) ATF_C(11) ATF_C(12) ATF_C(13) ATF_C(14) default: break; }
#undef ATF_C
    ATF_PAIR(NSTEP - 1);
#undef ATF_PAIR
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kPrefillWaves * 64, 8 / kPrefillWaves) void prefill_bf16_kernel(
    AttnArgs a) {
    constexpr int P = D / 2;
    constexpr int NW = kPrefillWaves;  // waves per workgroup (two per SIMD)
    constexpr int KT = kPrefillKeys;   // keys per LDS tile
    constexpr int QT = 32 * NW;           // queries per workgroup
    constexpr int NB = KT / 32;        // 32-key score blocks per tile
    constexpr int NSTEP = D / 16;      // MFMA K-steps of 16 dims (8 pairs)
    constexpr int CH = D / 8;          // 16-byte chunks per rotated-key row
    constexpr int NDB = D / 32;        // 32-dim blocks of the output
    constexpr unsigned KT_BYTES = KT * D * 2;
    constexpr unsigned TILE_BYTES = 2 * KT_BYTES;  // K' then V^T (KT/64 tiles of [D][64])
    constexpr int NLD = KT_BYTES / 1024 / NW;      // 1 KB direct loads per wave per tile (each of K', V^T)
    static_assert(NLD >= 1 && NB % 2 == 0, "tile shape");
    static_assert(D <= 128, "d = 256 has its own kernel");
    __shared__ __attribute__((aligned(1024))) unsigned char lds[2 * TILE_BYTES];

    // ---- work unit u = (key split sp, work item gi), split-major, longest
    // query tiles first within a split.  Workgroup ids are dealt to the 8 XCDs
    // round robin; unit u runs on XCD u % 8 with its group workgroups (the
    // heads sharing one kv head), so K/V tiles are reused in that XCD's L2;
    // when the work items do not fill the 8 XCDs, consecutive splits of a
    // short chunk go to the others.
    // A work item is QT query rows of one head (wave w: rows 32 w ..), or, head
    // packed (a.hpack, for short chunks), 32 query rows of up to NW heads that
    // share the kv head (wave w: head NW * slab + w of the group, the same
    // rows), so one LDS key tile serves NW heads; a.group then counts slabs.
    const int L = blockIdx.x;
    const int xcd = L & 7, slot = L >> 3;
    const int u = (slot / a.group) * 8 + xcd;
    if (u >= a.n_groups * a.n_ksplit) return;
    const int gi = u % a.n_groups, sp = u / a.n_groups;
    const int g = slot % a.group;
    const int per_qt = a.B * a.Hkv;
    const int qt = a.n_qtiles - 1 - gi / per_qt;
    const int rem = gi % per_qt;
    const int b = rem / a.Hkv, hk = rem % a.Hkv;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int qi = lane & 31, half = lane >> 5;
    const int hgroup = a.Hq / a.Hkv;
    const int hw = a.hpack ? NW * g + wave : 0;  // packed: head within the kv group
    const int h = a.hpack ? hk * hgroup + min(hw, hgroup - 1) : hk * a.group + g;
    const int QS = a.hpack ? 32 : QT;            // query rows of the work item
    const int i0 = a.hpack ? qt * 32 : qt * QT + wave * 32;  // first query row of this wave
    const int my_q = i0 + qi;
    const bool q_valid = my_q < a.Sq && hw < hgroup;
    // Causal tests and distances run in key-index units: query row i sits at
    // key index i + qoff (qoff = Sk - Sq > 0 when a prefix of cached keys
    // precedes the query chunk).
    const int qoff = (int)(a.q_pos0 - a.k_pos0);
    const int i0k = i0 + qoff, my_qk = my_q + qoff, q0k = qt * QS + qoff;
    const WaveWin<P> win = load_windows<P>(a.W);

    // ---- this lane's rotated, pre-scaled query in B-operand order: step s
    // holds pairs 8s + 4*half + (0..3), each as (x'_p, x'_{p+P}) * log2(e)/sqrt(d)
    bf16x8_t qf[NSTEP];
    {
        const unsigned short *qrow =
            (const unsigned short *)a.q + ((long long)(b * a.Hq + h) * a.Sq + my_q) * D;
        const long long pos = a.q_pos0 + my_q;
        const float sc = a.scale_log2;
#pragma unroll
        for (int s = 0; s < NSTEP; ++s) {
            u32x4 w = (u32x4){0u, 0u, 0u, 0u};
            if (q_valid) {
                const int p0 = 8 * s + 4 * half;
                u32x2 lo, hi;
                load_pair_pieces(qrow, p0, P, a.gptj != 0, lo, hi);
                unsigned r[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    float x, y, c, sn;
                    pair_xy(lo, hi, u, a.gptj != 0, x, y);
                    rope_cos_sin(pos, a.theta[p0 + u], c, sn);
                    r[u] = pack_bf((x * c - y * sn) * sc, (y * c + x * sn) * sc);
                }
                w = (u32x4){r[0], r[1], r[2], r[3]};
            }
            qf[s] = __builtin_bit_cast(bf16x8_t, w);
        }
    }

    const unsigned char *kg = (const unsigned char *)a.krot + (long long)(b * a.Hkv + hk) * a.Sk_pad * (D * 2);
    const unsigned char *vg = (const unsigned char *)a.vt + (long long)(b * a.Hkv + hk) * a.Sk_pad * (D * 2);
    // causal: keys up to the workgroup's last query; otherwise every key, the
    // windows applying to |i - j|
    const int last_key = CAUSAL ? min(a.Sk - 1, q0k + QS - 1) : a.Sk - 1;
    const int n_kt = last_key / KT + 1;
    // key tiles of this workgroup's split: kt0, kt0 + ks, ... below n_kt.  The
    // splits take the tiles in turn rather than contiguous ranges, so the
    // tiles near the queries, whose windows put boundary pairs and more kept
    // pairs in them and which cost up to several times a far tile, are
    // spread over all splits.
    const int kt0 = sp, ks = a.n_ksplit;

    // Direct global->LDS loads of tile kt into buffer buf.  Lane l of this
    // wave's n-th 1 KB piece lands at LDS byte piece*1024 + 16 l (lane-linear),
    // so the lane fetches the global chunk that the swizzle puts there.  Key
    // chunks whose pairs no block of this workgroup can use are not fetched
    // (c_min: first 16-byte chunk any wave reads in this tile).
    // Piece n of wave w is tile piece n*NW + w.  When the piece stride covers
    // whole swizzle periods every piece of a lane has the same swizzle (one
    // per-lane offset plus n * NW KB in a scalar); otherwise the lane has KPER
    // offsets, piece n using offset n % KPER.
    constexpr int KPERIOD = CH * 16 * kswz_rows<CH>();  // bytes of one key-swizzle period
    constexpr int KPER = (KPERIOD > NW * 1024) ? KPERIOD / (NW * 1024) : 1;
    static_assert((NW * 1024) % KPERIOD == 0 || KPERIOD % (NW * 1024) == 0, "piece stride vs key swizzle");
    // swz8 repeats every 16 value rows (2 KB)
    static_assert((NW * 1024) % (128 * 16) == 0, "a piece stride must keep the value-row swizzle");
    unsigned k_goff[KPER], v_goff;
    int k_chunk[KPER];
#pragma unroll
    for (int e = 0; e < KPER; ++e) {
        const int kbyte = (e * NW + wave) * 1024 + lane * 16;
        const int krow = kbyte / (CH * 16);
        k_chunk[e] = ((kbyte / 16) % CH) ^ kswz<CH>(krow);
        k_goff[e] = (unsigned)(krow * (CH * 16) + k_chunk[e] * 16) - (unsigned)(e * NW * 1024);
    }
    {
        const int kbyte = wave * 1024 + lane * 16;
        const int vrow = kbyte / 128;
        v_goff = (unsigned)(vrow * 128 + ((((kbyte / 16) & 7) ^ swz8(vrow)) * 16));
    }
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
#define ATF_TILE_LOAD(kt_, buf_, part_)                                                    \
    {                                                                                      \
        const int j0_ = (kt_) * KT;                                                        \
        const int dmin_wg_ = CAUSAL ? max(0, q0k - (j0_ + KT - 1))                         \
                                    : max(0, max(q0k - (j0_ + KT - 1), j0_ - (q0k + QS - 1))); \
        const int c_min_ = 2 * (cut_below(win, dmin_wg_) >> 3);                            \
        /* a key chunk below c_min is not fetched: its offset is past the buffer's end */ \
        unsigned koff_[KPER];                                                              \
        _Pragma("unroll") for (int e = 0; e < KPER; ++e)                                   \
            koff_[e] = (k_chunk[e] >= c_min_) ? k_goff[e] : KT_BYTES;                      \
        const __amdgpu_buffer_rsrc_t kr_ = raw_rsrc(kg + (long long)j0_ * (D * 2), KT_BYTES); \
        const __amdgpu_buffer_rsrc_t vr_ = raw_rsrc(vg + (long long)j0_ * (D * 2), KT_BYTES); \
        unsigned char *lk_ = lds + (buf_) * TILE_BYTES + wave_s * 1024;                    \
        _Pragma("unroll") for (int n = 0; n < NLD; ++n) {                                  \
            if ((part_) & 1) lds_dma16_buf(kr_, koff_[n % KPER], n * NW * 1024, lk_ + n * NW * 1024); \
            if ((part_) & 2) lds_dma16_buf(vr_, v_goff, n * NW * 1024, lk_ + KT_BYTES + n * NW * 1024); \
        }                                                                                  \
    }

    f32x16_t o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
    // Softmax reference m_ref (log2 units, a bf16 value) and running sum.  The
    // score MFMAs subtract m_ref, so a probability is 2^score.  m_ref moves
    // only at the first block and when a lane's sum over a block's 16 keys
    // exceeds kSumLimit (some probability above kSumLimit/16, or an overflow):
    // then the block's exact max becomes the reference and the block is redone.
    // Probabilities therefore stay below kSumLimit and the O rescale is rare.
    constexpr float kSumLimit = 4096.f;
    float m_ref = 0.f, l_run = 0.f;
    bool first = true;
    // rank-1 operands of the reference: element k = 0 of lanes 0..31 (A: ones
    // for every key row; B: -m_ref of the lane's query column), zeros elsewhere
    const s16x4_t ones_a = __builtin_bit_cast(s16x4_t, (u32x2){half ? 0u : 0x3f80u, 0u});
    s16x4_t negm_b = __builtin_bit_cast(s16x4_t, (u32x2){0u, 0u});
    // dropped-term count: per lane where it differs between lanes, uniform
    // (whole-block) contributions in skipped_u
    // (non-causal, at the register limit: a lane's boundary-term count fits
    // 32 bits, since a wave meets at most two general tiles per window plus
    // the diagonal and last ones, each adding at most 4 x 16 x P terms)
    using lane_cnt_t = std::conditional_t<CAUSAL, unsigned long long, unsigned>;
    lane_cnt_t skipped = 0;
    unsigned long long skipped_u = 0;
    unsigned fast_cut = 0;  // sum of the pair cut over fast tiles (x NB x 16 x n_valid at the end)
    const unsigned n_valid = (unsigned)__builtin_popcountll(__ballot(q_valid));
    const f32x16_t zero16 = {};
    const int koff0 = 4 * half;
    // non-causal (at the register limit): my_qk - koff0 recomputed from the
    // lane id where the boundary path needs it rather than held across the
    // tile loop; the empty move keeps the compiler from hoisting it back out
    auto nc_dq_base = [&]() {
        int z;
        asm volatile("v_mov_b32 %0, 0" : "=v"(z));
        const int ln = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, (unsigned)z));
        return i0k + (ln & 31) - 4 * (ln >> 5);
    };
    // per-lane LDS byte offsets (swizzle folded in)
    const unsigned krow0 = (unsigned)qi;  // key row of block 0; block 1 is +32 rows
    const unsigned kbase_lane = krow0 * (CH * 16);
    const unsigned ky = (unsigned)((kswz<CH>(qi) ^ half) << 4);
    const unsigned vbase_lane = KT_BYTES + (unsigned)qi * 128;
    const unsigned vz = (unsigned)((swz8(qi) ^ half) << 4);

    if (kt0 < n_kt) ATF_TILE_LOAD(kt0, 0, 3);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    for (int kt = kt0, it = 0; kt < n_kt; kt += ks, ++it) {
        const int buf = it & 1;
        const bool more = kt + ks < n_kt;
        const unsigned char *lt = lds + buf * TILE_BYTES;
        const int j0 = kt * KT;

        // Per pair of 32-key blocks: chain0 | chain1 + probs0 | PV0 + probs1 |
        // PV1, so every MFMA run but the first and last has independent VALU
        // work beside it.  Boundary pairs, diagonal masks and reference moves
        // sit between the runs (rare branches).
        f32x16_t sacc[2];
        unsigned pw[2][8];
        float lsum[2];

        // Move the reference when block kb's probabilities overflow kSumLimit
        // (or at the first block): block max becomes the reference, O and l are
        // rescaled, the block's probabilities are redone; the next block, already
        // scored against the old reference (when `later` holds), is shifted too.
#define ATF_BLOCK_RESCALE(sl, later)                                                              \
        if (__ballot(first || !(lsum[sl] <= kSumLimit))) {                                        \
            float bm = sacc[sl][0];                                                               \
            _Pragma("unroll") for (int r = 1; r < 16; ++r) bm = fmaxf(bm, sacc[sl][r]);           \
            bm = partner_max(bm);                                                                 \
            /* (first block: a query with all its keys masked keeps the reference) */              \
            const float m_new = first ? (bm == -INFINITY ? m_ref : bf16_ceil(m_ref + bm))          \
                                      : fmaxf(m_ref, bf16_ceil(m_ref + bm));                       \
            const float shift = m_new - m_ref;                                                    \
            if (!first) {                                                                         \
                const float corr = fast_exp2(-shift);                                             \
                l_run *= corr;                                                                    \
                _Pragma("unroll") for (int db = 0; db < NDB; ++db)                                \
                    _Pragma("unroll") for (int r = 0; r < 16; ++r) o[db][r] *= corr;              \
            }                                                                                     \
            m_ref = m_new;                                                                        \
            if (later) {                                                                          \
                _Pragma("unroll") for (int r = 0; r < 16; ++r) sacc[(sl) ^ 1][r] -= shift;        \
            }                                                                                     \
            negm_b = __builtin_bit_cast(s16x4_t, (u32x2){half ? 0u : (pack_bf(-m_ref, 0.f) & 0xffffu), 0u}); \
            _Pragma("unroll") for (int r = 0; r < 16; ++r) sacc[sl][r] -= shift;                  \
            block_probs(sacc[sl], pw[sl], lsum[sl]);                                              \
        }                                                                                         \
        first = false;                                                                            \
        l_run += lsum[sl];

        // Fast tile (the common case): for this wave every key of the tile
        // precedes every query (causal; non-causal also: follows every query,
        // none past the end) and no window W_p falls inside the tile's
        // distance range, so all its blocks keep the same pair suffix [p_t, P)
        // with no per-element work.
        bool fast;
        int p_t;
        {
            const int jl = j0 + KT - 1;
            int dmin, dmax;
            if (CAUSAL) {
                fast = jl <= i0k;
                dmin = i0k - jl;
                dmax = i0k + 31 - j0;
            } else {
                // every key of the tile on one side of every query of the
                // wave, none past the end: distances |i - j| span [dmin, dmax]
                const bool before = jl <= i0k, after = j0 > i0k + 31;
                fast = (before || after) && jl < a.Sk;
                dmin = before ? i0k - jl : j0 - (i0k + 31);
                dmax = before ? i0k + 31 - j0 : jl - i0k;
            }
            const int plo_t = cut_below(win, dmin);
            p_t = cut_below(win, dmax);
            fast = fast && plo_t == p_t;
        }
        // The next tile's loads: on fast tiles its keys after the first block
        // pair's score chains and its values after that pair, rather than
        // both at the tile start, where every wave's first chains read the
        // keys of this tile.
        if (fast) {
            fast_cut += (unsigned)p_t;
            const int sf = p_t >> 3, zb = p_t - 8 * sf - koff0;
#pragma unroll
            for (int kp = 0; kp < NB; kp += 2) {
                if (NB > 2 && kp == 2 && more) ATF_TILE_LOAD(kt + ks, buf ^ 1, 2);
                const unsigned char *lv = lt + (kp >> 1) * (D * 128);
                qk_pair<NSTEP>(sf, lt, kbase_lane + 32u * kp * (CH * 16), kbase_lane + 32u * (kp + 1) * (CH * 16), ky,
                               qf, zb, ones_a, negm_b, sacc[0], sacc[1], pw[0], lsum[0]);
                // (a one-pair tile takes its values here too)
                if (kp == 0 && more) ATF_TILE_LOAD(kt + ks, buf ^ 1, NB > 2 ? 1 : 3);
                ATF_BLOCK_RESCALE(0, true)
                block_pv<NDB>(o, lv, vbase_lane, vz, 0, pw[0]);
                block_probs(sacc[1], pw[1], lsum[1]);
                ATF_BLOCK_RESCALE(1, false)
                block_pv<NDB>(o, lv, vbase_lane, vz, 1, pw[1]);
            }
            __builtin_amdgcn_s_waitcnt(0);  // this wave's direct loads of the next tile
            __syncthreads();
            continue;
        }

        if (more) ATF_TILE_LOAD(kt + ks, buf ^ 1, 3);
        int p_lo[NB], p_full[NB];
        bool live[NB];
#pragma unroll
        for (int kb = 0; kb < NB; ++kb) {
            const int jb = j0 + 32 * kb;
            // distances i - j of the block span [i0k - jb - 31, i0k + 31 - jb]
            const int dlo = i0k - jb - 31, dhi = i0k + 31 - jb;
            live[kb] = CAUSAL ? dhi >= 0 : jb < a.Sk;
            const int amin = CAUSAL ? max(0, dlo) : max(0, max(dlo, -dhi));
            const int amax = CAUSAL ? dhi : max(dhi, -dlo);
            p_lo[kb] = cut_below(win, amin);
            p_full[kb] = cut_below(win, amax);
        }

        // boundary pairs (one rank-2 MFMA each, added where the distance is
        // inside W_p), dropped-term count and causal mask of block kb (slot sl)
#define ATF_BLOCK_EDGES(kb, sl)                                                                   \
        {                                                                                         \
            const int jb = j0 + 32 * (kb);                                                        \
            /* causal: some key may follow some query; otherwise: some key is past Sk */          \
            const bool diag = CAUSAL ? jb + 31 > i0k : jb + 31 >= a.Sk;                           \
            const unsigned kbase = kbase_lane + 32u * (kb) * (CH * 16);                           \
            /* element r holds key jb + koff0 + c_r, c_r = 8(r/4) + r%4, at distance dq - c_r;    \
               it is a real (causal) key iff c_r < vlim */                                        \
            const int dq = (CAUSAL ? my_qk - koff0 : nc_dq_base()) - jb;                          \
            const int vlim = CAUSAL ? dq + 1 : a.Sk - jb - koff0;                                 \
            if (p_lo[kb] > 0) {                                                                   \
                if (!diag) {                                                                      \
                    skipped_u += (unsigned long long)p_lo[kb] * 16u * n_valid;                    \
                } else if (q_valid) {                                                             \
                    skipped += (lane_cnt_t)p_lo[kb] * (unsigned)keys_below(vlim);                 \
                }                                                                                 \
            }                                                                                     \
            if (p_lo[kb] < p_full[kb]) {                                                          \
                _Pragma("unroll") for (int s = 0; s < NSTEP; ++s) {                               \
                    const int pa = max(p_lo[kb], 8 * s), pe = min(p_full[kb], 8 * s + 8);         \
                    if (pa < pe) {                                                                \
                        const u32x4 kraw = *(const u32x4 *)(lt + kbase + ((32u * s) ^ ky));       \
                        const int pb = 8 * s + koff0;                                             \
                        for (int p = pa; p < pe; ++p) {                                           \
                            u32x4 kw;                                                             \
                            kw.x = (pb + 0 == p) ? kraw.x : 0u;                                   \
                            kw.y = (pb + 1 == p) ? kraw.y : 0u;                                   \
                            kw.z = (pb + 2 == p) ? kraw.z : 0u;                                   \
                            kw.w = (pb + 3 == p) ? kraw.w : 0u;                                   \
                            const f32x16_t tp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(          \
                                __builtin_bit_cast(bf16x8_t, kw), qf[s], zero16, 0, 0, 0);        \
                            /* pair p is kept iff |dq - c_r| <= W_p: lim <= c_r <= him */      \
                            const int wp = window_at(win, p);                                     \
                            const int lim = dq - wp, him = CAUSAL ? dq : dq + wp;                 \
                            _Pragma("unroll") for (int r = 0; r < 16; ++r) {                      \
                                const int c = 8 * (r >> 2) + (r & 3);                             \
                                sacc[sl][r] += (c >= lim && (CAUSAL || c <= him)) ? tp[r] : 0.f;  \
                            }                                                                     \
                            if (q_valid)                                                          \
                                skipped += (unsigned)(keys_below(min(lim, vlim)) +                \
                                                      (CAUSAL ? 0 : keys_below(vlim) -           \
                                                                     keys_below(min(vlim, him + 1)))); \
                        }                                                                         \
                    }                                                                             \
                }                                                                                 \
            }                                                                                     \
            if (diag) {                                                                           \
                _Pragma("unroll") for (int r = 0; r < 16; ++r)                                    \
                    if (8 * (r >> 2) + (r & 3) >= vlim) sacc[sl][r] = -INFINITY;                  \
            }                                                                                     \
        }


#pragma unroll
        for (int kp = 0; kp < NB; kp += 2) {  // pairs of blocks: slot 0 = block kp, slot 1 = kp + 1
            if (!live[kp]) break;
            const unsigned char *lv = lt + (kp >> 1) * (D * 128);  // the pair's 64-key V^T tile
            const int sf0 = p_full[kp] >> 3;
            sacc[0] = qk_main<NSTEP>(sf0, lt, kbase_lane + 32u * kp * (CH * 16), ky, qf,
                                     p_full[kp] - 8 * sf0 - koff0, ones_a, negm_b);
            ATF_BLOCK_EDGES(kp, 0)
            const bool live1 = live[kp + 1];
            if (live1) {
                const int sf1 = p_full[kp + 1] >> 3;
                sacc[1] = qk_main_probs<NSTEP>(sf1, lt, kbase_lane + 32u * (kp + 1) * (CH * 16), ky, qf,
                                               p_full[kp + 1] - 8 * sf1 - koff0, ones_a, negm_b, sacc[0], pw[0],
                                               lsum[0]);
            } else {
                block_probs(sacc[0], pw[0], lsum[0]);
            }
            ATF_BLOCK_RESCALE(0, live1)
            if (live1) {
                ATF_BLOCK_EDGES(kp + 1, 1)
                block_pv<NDB>(o, lv, vbase_lane, vz, 0, pw[0]);
                block_probs(sacc[1], pw[1], lsum[1]);
                ATF_BLOCK_RESCALE(1, false)
                block_pv<NDB>(o, lv, vbase_lane, vz, 1, pw[1]);
            } else {
                block_pv<NDB>(o, lv, vbase_lane, vz, 0, pw[0]);
            }
        }
#undef ATF_BLOCK_EDGES
#undef ATF_BLOCK_RESCALE

        __builtin_amdgcn_s_waitcnt(0);  // this wave's direct loads of the next tile
        __syncthreads();
    }
#undef ATF_TILE_LOAD

    // ---- epilogue: O / l, bf16, store (lane holds dims 32db + 8g + 4*half + 0..3).
    // A key-range split instead writes its unnormalised O, m_ref and l (m =
    // -inf when the split holds none of the query's mass) for the combine.
    // Non-causal (at the register limit): the row and head are recomputed
    // from the lane id and the uniform wave index, so no per-lane prologue
    // value stays live across its tile loop.
    const float l_tot = partner_sum(l_run);
    {
    const int lane_e = CAUSAL ? lane : (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    const int half_e = CAUSAL ? half : lane_e >> 5;
    const int hw_e = a.hpack ? NW * g + wave_s : 0;
    const int h_e = CAUSAL ? h : a.hpack ? hk * hgroup + min(hw_e, hgroup - 1) : hk * a.group + g;
    const int my_q_e = CAUSAL ? my_q : (a.hpack ? qt * 32 : qt * QT + wave_s * 32) + (lane_e & 31);
    const bool q_valid_e = CAUSAL ? q_valid : my_q_e < a.Sq && hw_e < hgroup;
    if (a.n_ksplit > 1) {
        if (q_valid_e) {
            float *pr = a.part + ((((long long)(b * a.Hq + h_e) * a.Sq + my_q_e) * a.n_ksplit) + sp) * (D + 2);
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {  // rows of d + 2 floats are 8-byte aligned
                    float *pd = pr + 32 * db + 8 * g4 + 4 * half_e;
                    *(float2 *)pd = make_float2(o[db][4 * g4], o[db][4 * g4 + 1]);
                    *(float2 *)(pd + 2) = make_float2(o[db][4 * g4 + 2], o[db][4 * g4 + 3]);
                }
            if (half_e == 0) {
                pr[D] = l_tot > 0.f ? m_ref : -INFINITY;
                pr[D + 1] = l_tot;
            }
        }
    } else if (q_valid_e) {
        const float inv = 1.f / l_tot;
        unsigned short *orow = (unsigned short *)a.out + ((long long)(b * a.Hq + h_e) * a.Sq + my_q_e) * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                u32x2 w;
                w.x = pack_bf(o[db][4 * g4 + 0] * inv, o[db][4 * g4 + 1] * inv);
                w.y = pack_bf(o[db][4 * g4 + 2] * inv, o[db][4 * g4 + 3] * inv);
                *(u32x2 *)(orow + 32 * db + 8 * g4 + 4 * half_e) = w;
            }
    }
    skipped_u += (unsigned long long)fast_cut * (NB * 16u) * n_valid;
    const unsigned long long total = wave_sum_u64((unsigned long long)skipped) + skipped_u;
    if (lane_e == 0 && total) atomicAdd(a.counter, total);
    }
}

// ============================================================================
// Prefill attention, bf16 in / fp32 accumulate, MFMA 16x16x32: the d = 256
// kernel (written for d = 128 or 256; at d = 128 the 32x32 kernel above is
// faster, since here P.V reads V^T from LDS at twice the rate per flop).
//
// Workgroup = 8 waves (two per SIMD) = 128 queries of one (b, h); wave w owns
// 16 queries, so its accumulators (16 x 256 fp32) and query fragments fit two
// waves per SIMD.  Key tiles (64 keys at d = 256) stream into LDS with direct
// loads from the same prepared K' / V^T as the 32x32 kernel, double-buffered,
// one barrier per tile.  Per 32-key block a wave computes two 16x16 score
// blocks S^T = K' Q'^T (sub-block sb: MFMA row t is key 2(t & 8) + (t & 7) +
// 8 sb of the block) over the kept 32-dim K-steps (16 pairs each), then
// O^T[16 dims x 16 queries] += V^T P^T for every 16-dim output block.  Lane
// (t, g) = (lane % 16, lane / 16) owns query t; its score rows 4g + r (r =
// 0..3) of sub-block sb are key 16(g >> 1) + 4(g & 1) + 8 sb + r, exactly
// the keys the value tile's in-group permutation puts in that lane's P.V
// operand, so the four probability words are the operand as they stand.
//
// Windows, fast tiles, boundary pairs, masks and counting follow the 32x32
// kernel, on 16-pair K-steps: pairs below the cut inside the first kept step
// are zeroed on the query side (once per tile on the fast path).  The softmax
// reference enters as the initial accumulator: every element of a lane's
// 16x16 score block belongs to its one query, so {-m_ref x 4} is the C
// operand of the first score MFMA and a probability is 2^score.
// ============================================================================

// K' LDS swizzle of the 16x16 kernel: the 16 rows one 16-lane group reads
// (keys 0..7 and 16..23 of a block, or 8..15 and 24..31) get 16 distinct
// 16-byte bank groups, for 256- and 512-byte rows alike.
__device__ inline int kswz_sub(int row) { return (row & 7) | (((row >> 4) & 1) << 3); }

// keys of the lane's 8 score slots below x (slot (sb, r): key base_g + 8 sb + r)
__device__ inline int slots_below16(int x, int base_g) {
    return min(max(x - base_g, 0), 4) + min(max(x - base_g - 8, 0), 4);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kPrefill16Waves * 64, kPrefill16Waves / 4) void prefill16_bf16_kernel(AttnArgs a) {
    constexpr int P = D / 2;
    constexpr int NW = kPrefill16Waves;
    constexpr int KT = D == 256 ? kPrefill16Keys : 128;
    constexpr int QT = 16 * NW;
    constexpr int NB = KT / 32;
    constexpr int NSTEP = D / 32;  // K-steps of 32 dims (16 pairs)
    constexpr int CH = D / 8;      // 16-byte chunks per K' row
    constexpr int NDB = D / 16;    // 16-dim output blocks
    constexpr unsigned KT_BYTES = KT * D * 2;
    constexpr unsigned TILE_BYTES = 2 * KT_BYTES;
    constexpr int NPIECE = KT_BYTES / 1024;            // 1 KB pieces per tile (each of K', V^T)
    constexpr int NLD = (NPIECE + NW - 1) / NW;        // pieces per wave
    static_assert(D == 128 || D == 256, "16x16 prefill: d = 128 or 256");
    static_assert(NW % 2 == 0, "swz8 repeats every 16 value rows (2 KB): the piece stride must keep it");
    __shared__ __attribute__((aligned(1024))) unsigned char lds[2 * TILE_BYTES];

    const int L = blockIdx.x;  // work units and XCD placement as in the 32x32 kernel
    const int xcd = L & 7, slot = L >> 3;
    const int u = (slot / a.group) * 8 + xcd;
    if (u >= a.n_groups * a.n_ksplit) return;
    const int gi = u % a.n_groups, sp = u / a.n_groups;
    const int hs = slot % a.group;  // head in the group, or (head packed) slab of NW heads
    const int per_qt = a.B * a.Hkv;
    const int qt = a.n_qtiles - 1 - gi / per_qt;
    const int rem = gi % per_qt;
    const int b = rem / a.Hkv, hk = rem % a.Hkv;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int t = lane & 15, g = lane >> 4;
    // as in the 32x32 kernel: QT rows of one head, or 16 rows of NW heads
    const int hgroup = a.Hq / a.Hkv;
    const int hw = a.hpack ? NW * hs + wave : 0;
    const int h = a.hpack ? hk * hgroup + min(hw, hgroup - 1) : hk * a.group + hs;
    const int QS = a.hpack ? 16 : QT;
    const int i0 = a.hpack ? qt * 16 : qt * QT + wave * 16;
    const int my_q = i0 + t;
    const bool q_valid = my_q < a.Sq && hw < hgroup;
    const int qoff = (int)(a.q_pos0 - a.k_pos0);
    const int i0k = i0 + qoff, my_qk = my_q + qoff, q0k = qt * QS + qoff;
    const WaveWin<P> win = load_windows<P>(a.W);
    const int kbase_g = 16 * (g >> 1) + 4 * (g & 1);  // key of slot (sb 0, r 0) in a block

    // query operand: step s holds pairs 16 s + 4 g + (0..3) of query t, rotated and scaled
    // (read from a.qrot when the call rotated the queries once beforehand)
    bf16x8_t qf[NSTEP];
    if (a.qrot) {
        const unsigned *qr = a.qrot + ((long long)(b * a.Hq + h) * a.Sq + my_q) * P;
#pragma unroll
        for (int s = 0; s < NSTEP; ++s) {
            u32x4 w = (u32x4){0u, 0u, 0u, 0u};
            if (q_valid) w = *(const u32x4 *)(qr + 16 * s + 4 * g);
            qf[s] = __builtin_bit_cast(bf16x8_t, w);
        }
    } else {
        const unsigned short *qrow = (const unsigned short *)a.q + ((long long)(b * a.Hq + h) * a.Sq + my_q) * D;
        const long long pos = a.q_pos0 + my_q;
        const float sc = a.scale_log2;
#pragma unroll
        for (int s = 0; s < NSTEP; ++s) {
            u32x4 w = (u32x4){0u, 0u, 0u, 0u};
            if (q_valid) {
                const int p0 = 16 * s + 4 * g;
                u32x2 lo, hi;
                load_pair_pieces(qrow, p0, P, a.gptj != 0, lo, hi);
                unsigned r[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    float x, y, c, sn;
                    pair_xy(lo, hi, u, a.gptj != 0, x, y);
                    rope_cos_sin(pos, a.theta[p0 + u], c, sn);
                    r[u] = pack_bf((x * c - y * sn) * sc, (y * c + x * sn) * sc);
                }
                w = (u32x4){r[0], r[1], r[2], r[3]};
            }
            qf[s] = __builtin_bit_cast(bf16x8_t, w);
        }
    }

    const unsigned char *kg = (const unsigned char *)a.krot + (long long)(b * a.Hkv + hk) * a.Sk_pad * (D * 2);
    const unsigned char *vg = (const unsigned char *)a.vt + (long long)(b * a.Hkv + hk) * a.Sk_pad * (D * 2);
    const int last_key = CAUSAL ? min(a.Sk - 1, q0k + QS - 1) : a.Sk - 1;
    const int n_kt = last_key / KT + 1;
    // key tiles of this workgroup's split: kt0, kt0 + ks, ... below n_kt.  The
    // splits take the tiles in turn rather than contiguous ranges, so the
    // tiles near the queries, whose windows put boundary pairs and more kept
    // pairs in them and which cost up to several times a far tile, are
    // spread over all splits.
    const int kt0 = sp, ks = a.n_ksplit;

    // Tile loader: piece m (1 KB) of K' lands lane-linear at LDS byte 1024 m +
    // 16 l, i.e. row (1024 m + 16 l) / row_bytes, physical chunk l % CH; the
    // lane fetches the logical chunk the swizzle maps there (chunks below
    // c_min, whose pairs the whole workgroup drops, read past the buffer end
    // and land as zeros).  V^T pieces keep one per-lane offset: the piece
    // stride NW KB is a whole number of value-swizzle periods.
    unsigned v_goff;
    {
        const int kbyte = wave * 1024 + lane * 16;
        const int vrow = kbyte / 128;
        v_goff = (unsigned)(vrow * 128 + ((((kbyte / 16) & 7) ^ swz8(vrow)) * 16));
    }
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
#define ATF16_TILE_LOAD(kt_, buf_)                                                           \
    {                                                                                      \
        const int j0_ = (kt_) * KT;                                                        \
        const int dmin_wg_ = CAUSAL ? max(0, q0k - (j0_ + KT - 1))                         \
                                    : max(0, max(q0k - (j0_ + KT - 1), j0_ - (q0k + QS - 1))); \
        const int c_min_ = cut_below(win, dmin_wg_) >> 2;                                  \
        const __amdgpu_buffer_rsrc_t kr_ = raw_rsrc(kg + (long long)j0_ * (D * 2), KT_BYTES); \
        const __amdgpu_buffer_rsrc_t vr_ = raw_rsrc(vg + (long long)j0_ * (D * 2), KT_BYTES); \
        unsigned char *lk_ = lds + (buf_) * TILE_BYTES;                                    \
        _Pragma("unroll") for (int n = 0; n < NLD; ++n) {                                  \
            const int m_ = n * NW + wave_s;                                                \
            if (NPIECE % NW == 0 || m_ < NPIECE) {                                         \
                const int krow_ = (1024 * m_ + 16 * lane) / (CH * 16);                     \
                const int kch_ = (lane % CH) ^ kswz_sub(krow_);                               \
                const unsigned koff_ = kch_ >= c_min_ ? (unsigned)(kch_ * 16 + (lane / CH) * (CH * 16)) : KT_BYTES; \
                lds_dma16_buf(kr_, koff_, m_ * 1024, lk_ + m_ * 1024);                     \
                lds_dma16_buf(vr_, v_goff, n * NW * 1024, lk_ + KT_BYTES + wave_s * 1024 + n * NW * 1024); \
            }                                                                              \
        }                                                                                  \
    }

    f32x4_t o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[db] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    constexpr float kSumLimit = 4096.f;
    float m_ref = 0.f, l_run = 0.f;
    bool first = true;
    // -m_ref in every element: the first score MFMA of a block starts from it,
    // so scores leave the chain shifted by the reference (a lane's 4 elements
    // all belong to its query t)
    f32x4_t negm = {0.f, 0.f, 0.f, 0.f};
    // a lane's boundary-term count fits 32 bits: a wave meets at most two
    // general tiles per window plus the diagonal and last ones, each adding
    // at most 2 x 8 x P terms
    unsigned skipped = 0;
    unsigned long long skipped_u = 0;
    unsigned fast_cut = 0;
    const unsigned nq = (unsigned)__builtin_popcountll(__ballot(q_valid && g == 0));
    const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
    // per-lane LDS byte offsets: K' row of MFMA row t in sub-block sb of block
    // kb is 32 kb + 2(t & 8) + (t & 7) + 8 sb; V^T row of output block db is 16 db + t
    const int krow_t = 2 * (t & 8) + (t & 7);
    const unsigned ksw0 = (unsigned)kswz_sub(krow_t), ksw1 = (unsigned)kswz_sub(krow_t + 8);
    const unsigned vrow_base = KT_BYTES + (unsigned)t * 128;

    if (kt0 < n_kt) ATF16_TILE_LOAD(kt0, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    for (int kt = kt0, it = 0; kt < n_kt; kt += ks, ++it) {
        const int buf = it & 1;
        if (kt + ks < n_kt) ATF16_TILE_LOAD(kt + ks, buf ^ 1);
        const unsigned char *lt = lds + buf * TILE_BYTES;
        const int j0 = kt * KT;

        // key fragment of step s, sub-block sb, block kb (chunk 4 s + g)
        auto kfrag = [&](int kb, int sb, int s) -> u32x4 {
            const unsigned row = 32u * kb + krow_t + 8u * sb;
            const unsigned sw = sb ? ksw1 : ksw0;
            return *(const u32x4 *)(lt + row * (CH * 16) + (((unsigned)(4 * s + g) ^ sw) << 4));
        };
        // query operand of step s (an index known at compile time, so the
        // fragments stay in registers) with the lane's pairs below the cut zeroed
        auto qmask = [&](int s, int zb) -> bf16x8_t {
            u32x4 w = __builtin_bit_cast(u32x4, qf[s]);
            w.x = (0 < zb) ? 0u : w.x;
            w.y = (1 < zb) ? 0u : w.y;
            w.z = (2 < zb) ? 0u : w.z;
            w.w = (3 < zb) ? 0u : w.w;
            return __builtin_bit_cast(bf16x8_t, w);
        };
        // scores of block kb over steps s0..NSTEP-1 (s0 known at compile time;
        // step s0 with the query masked below the cut, zb)
        auto scores = [&](int kb, int s0, int zb, f32x4_t &c0, f32x4_t &c1) {
            c0 = negm;
            c1 = negm;
#pragma unroll
            for (int s = 0; s < NSTEP; ++s) {
                if (s < s0) continue;
                const u32x4 k0 = kfrag(kb, 0, s), k1 = kfrag(kb, 1, s);
                const bf16x8_t qs = (s == s0) ? qmask(s, zb) : qf[s];
                c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, k0), qs, c0, 0, 0, 0);
                c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, k1), qs, c1, 0, 0, 0);
            }
        };
        // the sum in fp32 before the rounding, as in the 32x32 kernel's block_probs
        auto probs = [&](const f32x4_t &c0, const f32x4_t &c1, u32x4 &pw, float &ls) {
            float e[8];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                e[r] = fast_exp2(c0[r]);
                e[4 + r] = fast_exp2(c1[r]);
            }
            pw.x = pack_bf(e[0], e[1]);
            pw.y = pack_bf(e[2], e[3]);
            pw.z = pack_bf(e[4], e[5]);
            pw.w = pack_bf(e[6], e[7]);
            ls = ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
        };
        // move the reference when a lane's block sum overflows (or at the first block)
        auto rescale = [&](f32x4_t &c0, f32x4_t &c1, u32x4 &pw, float &ls) {
            if (__ballot(first || !(ls <= kSumLimit))) {
                float bm = fmaxf(fmaxf(fmaxf(c0[0], c0[1]), fmaxf(c0[2], c0[3])),
                                 fmaxf(fmaxf(c1[0], c1[1]), fmaxf(c1[2], c1[3])));
                bm = quad_max(bm);  // block max relative to m_ref
                // (first block: a query with all its keys masked keeps the reference)
                const float m_new = first ? (bm == -INFINITY ? m_ref : m_ref + bm) : fmaxf(m_ref, m_ref + bm);
                const float shift = m_new - m_ref;
                if (!first) {
                    const float corr = fast_exp2(-shift);
                    l_run *= corr;
#pragma unroll
                    for (int db = 0; db < NDB; ++db) o[db] *= corr;
                }
                m_ref = m_new;
                negm = (f32x4_t){-m_ref, -m_ref, -m_ref, -m_ref};
                c0 -= shift;
                c1 -= shift;
                probs(c0, c1, pw, ls);
            }
            first = false;
            l_run += ls;
        };
        auto pv = [&](int kb, const u32x4 &pw) {
            const unsigned char *lv = lt + (kb >> 1) * (D * 128);
            const unsigned ch = (unsigned)(4 * (kb & 1) + g);
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const unsigned row = 16u * db + (unsigned)t;
                const u32x4 vf = *(const u32x4 *)(lv + vrow_base + 16u * db * 128 + ((ch ^ (unsigned)swz8((int)row)) << 4));
                o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, vf),
                                                                __builtin_bit_cast(bf16x8_t, pw), o[db], 0, 0, 0);
            }
        };

        bool fast;
        int p_t;
        {
            const int jl = j0 + KT - 1;
            if (CAUSAL) {
                fast = jl <= i0k;
                p_t = cut_below(win, i0k + 15 - j0);
                fast = fast && cut_below(win, i0k - jl) == p_t;
            } else {
                fast = false;
                p_t = 0;
            }
        }
        if (CAUSAL && fast) {
            fast_cut += (unsigned)p_t;
            const int sf = p_t >> 4, zb = p_t - 16 * sf - 4 * g;
            auto tile = [&](auto s0c) {
                constexpr int S0 = decltype(s0c)::value;
#pragma unroll
                for (int kb = 0; kb < NB; ++kb) {
                    f32x4_t c0, c1;
                    u32x4 pw;
                    float ls;
                    scores(kb, S0, zb, c0, c1);
                    probs(c0, c1, pw, ls);
                    rescale(c0, c1, pw, ls);
                    pv(kb, pw);
                }
            };
            // one case per K-step; the slowest pair is never cut, so sf < NSTEP
#define ATF16_T(i) \
                case i: if constexpr ((i) < NSTEP) tile(std::integral_constant<int, ((i) < NSTEP ? (i) : 0)>{}); break;
            switch (min(sf, NSTEP - 1)) {
                ATF16_T(0) ATF16_T(1) ATF16_T(2) ATF16_T(3) ATF16_T(4) ATF16_T(5) ATF16_T(6) ATF16_T(7)
                default: break;
            }
#undef ATF16_T
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            continue;
        }

#pragma unroll
        for (int kb = 0; kb < NB; ++kb) {
            const int jb = j0 + 32 * kb;
            const int dlo = i0k - jb - 31, dhi = i0k + 15 - jb;
            const bool live = CAUSAL ? dhi >= 0 : jb < a.Sk;
            if (!live) break;
            const int amin = CAUSAL ? max(0, dlo) : max(0, max(dlo, -dhi));
            const int amax = CAUSAL ? dhi : max(dhi, -dlo);
            const int p_lo = cut_below(win, amin), p_full = cut_below(win, amax);
            const bool diag = CAUSAL ? jb + 31 > i0k : jb + 31 >= a.Sk;
            const int dq = my_qk - jb;  // slot (sb, r) sits at distance dq - (kbase_g + 8 sb + r)
            const int vlim = CAUSAL ? dq + 1 : a.Sk - jb;  // slot keys below vlim are real keys
            f32x4_t c0, c1;
            const int sf = p_full >> 4, zb = p_full - 16 * sf - 4 * g;
#define ATF16_S(i) \
                case i: if constexpr ((i) < NSTEP) scores(kb, (i), zb, c0, c1); break;
            switch (min(sf, NSTEP - 1)) {
                ATF16_S(0) ATF16_S(1) ATF16_S(2) ATF16_S(3) ATF16_S(4) ATF16_S(5) ATF16_S(6) ATF16_S(7)
                default: break;
            }
#undef ATF16_S
            if (p_lo > 0) {
                if (!diag) skipped_u += (unsigned long long)p_lo * 32u * nq;
                else if (q_valid) skipped += (unsigned)p_lo * (unsigned)slots_below16(vlim, kbase_g);
            }
            // boundary pairs, step by step so each step's query fragment is a
            // register known at compile time
#pragma unroll
            for (int s = 0; s < NSTEP; ++s)
            for (int p = max(p_lo, 16 * s); p < min(p_full, 16 * s + 16); ++p) {
                const int gp = (p >> 2) & 3, w = p & 3;
                // (an opaque zero in the address keeps these reads from being
                // merged with the score chain's reads of the same step)
                int z;
                asm volatile("v_mov_b32 %0, 0" : "=v"(z));
                u32x4 k0 = kfrag(kb, 0, s + z), k1 = kfrag(kb, 1, s + z);
                const bool mine = g == gp;
                k0.x = (mine && w == 0) ? k0.x : 0u; k1.x = (mine && w == 0) ? k1.x : 0u;
                k0.y = (mine && w == 1) ? k0.y : 0u; k1.y = (mine && w == 1) ? k1.y : 0u;
                k0.z = (mine && w == 2) ? k0.z : 0u; k1.z = (mine && w == 2) ? k1.z : 0u;
                k0.w = (mine && w == 3) ? k0.w : 0u; k1.w = (mine && w == 3) ? k1.w : 0u;
                const bf16x8_t qs = qf[s];
                const f32x4_t t0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, k0), qs, zero4, 0, 0, 0);
                const f32x4_t t1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, k1), qs, zero4, 0, 0, 0);
                // pair p is kept at slot key c iff |dq - c| <= W_p: lim <= c (<= him)
                const int wp = window_at(win, p);
                const int lim = dq - wp, him = CAUSAL ? dq : dq + wp;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int ca = kbase_g + r, cb = kbase_g + 8 + r;
                    c0[r] += (ca >= lim && (CAUSAL || ca <= him)) ? t0[r] : 0.f;
                    c1[r] += (cb >= lim && (CAUSAL || cb <= him)) ? t1[r] : 0.f;
                }
                if (q_valid)
                    skipped += (unsigned)(slots_below16(min(lim, vlim), kbase_g) +
                                          (CAUSAL ? 0 : slots_below16(vlim, kbase_g) -
                                                            slots_below16(min(vlim, him + 1), kbase_g)));
            }
            if (diag) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    if (kbase_g + r >= vlim) c0[r] = -INFINITY;
                    if (kbase_g + 8 + r >= vlim) c1[r] = -INFINITY;
                }
            }
            u32x4 pw;
            float ls;
            probs(c0, c1, pw, ls);
            rescale(c0, c1, pw, ls);
            pv(kb, pw);
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }
#undef ATF16_TILE_LOAD

    // epilogue: lane (t, g) holds dims 16 db + 4 g + (0..3) of query t; a
    // key-range split writes its unnormalised O, m_ref and l for the combine.
    // The row and head are recomputed from the lane id and the uniform wave
    // index, so no per-lane prologue value stays live across the tile loop.
    const float l_tot = quad_sum(l_run);
    {
    const int lane_e = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    const int t_e = lane_e & 15, g_e = lane_e >> 4;
    const int hw_e = a.hpack ? NW * hs + wave_s : 0;
    const int h_e = a.hpack ? hk * hgroup + min(hw_e, hgroup - 1) : hk * a.group + hs;
    const int my_q_e = (a.hpack ? qt * 16 : qt * QT + wave_s * 16) + t_e;
    const bool q_valid_e = my_q_e < a.Sq && hw_e < hgroup;
    if (a.n_ksplit > 1) {
        if (q_valid_e) {
            float *pr = a.part + ((((long long)(b * a.Hq + h_e) * a.Sq + my_q_e) * a.n_ksplit) + sp) * (D + 2);
#pragma unroll
            for (int db = 0; db < NDB; ++db) {  // rows of d + 2 floats are 8-byte aligned
                *(float2 *)(pr + 16 * db + 4 * g_e) = make_float2(o[db][0], o[db][1]);
                *(float2 *)(pr + 16 * db + 4 * g_e + 2) = make_float2(o[db][2], o[db][3]);
            }
            if (g_e == 0) {
                pr[D] = l_tot > 0.f ? m_ref : -INFINITY;
                pr[D + 1] = l_tot;
            }
        }
    } else if (q_valid_e) {
        const float inv = 1.f / l_tot;
        unsigned short *orow = (unsigned short *)a.out + ((long long)(b * a.Hq + h_e) * a.Sq + my_q_e) * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            u32x2 w;
            w.x = pack_bf(o[db][0] * inv, o[db][1] * inv);
            w.y = pack_bf(o[db][2] * inv, o[db][3] * inv);
            *(u32x2 *)(orow + 16 * db + 4 * g_e) = w;
        }
    }
    skipped_u += (unsigned long long)fast_cut * (NB * 32u) * nq;
    const unsigned long long total = wave_sum_u64((unsigned long long)skipped) + skipped_u;
    if (lane_e == 0 && total) atomicAdd(a.counter, total);
    }
}

// ============================================================================
// fp32 attention (prefill and decode): plain VALU, one query per lane, keys
// rotated on the fly per 32-key LDS tile, exact per-element window test.
// Serves the fp32 dtype (parity workloads), not the bf16 hot path.
// grid (ceil(Sq/64), B*Hq), block 64.
// ============================================================================

template <int D>
__global__ __launch_bounds__(64) void attend_f32_kernel(AttnArgs a) {
    constexpr int P = D / 2;
    constexpr int TK = 32;
    __shared__ float2 ks[TK][P];
    __shared__ float vs[TK][D];
    const int bh = blockIdx.y;
    const int b = bh / a.Hq, h = bh % a.Hq, hk = h / a.group;
    const int lane = threadIdx.x;
    const int qblk0 = blockIdx.x * 64;
    const int i = qblk0 + lane;
    const bool valid = i < a.Sq;
    const long long qpos = a.q_pos0 + i;

    float qx[P], qy[P];
    {
        const float *qrow = (const float *)a.q + ((long long)bh * a.Sq + (valid ? i : 0)) * D;
#pragma unroll
        for (int p = 0; p < P; ++p) {
            float c, s;
            rope_cos_sin(qpos, a.theta[p], c, s);
            const int il = a.gptj ? 2 * p : p, ih = a.gptj ? 2 * p + 1 : p + P;  // the pair's two dims
            const float x = valid ? qrow[il] : 0.f, y = valid ? qrow[ih] : 0.f;
            qx[p] = x * c - y * s;
            qy[p] = y * c + x * s;
        }
    }
    const float *kh = (const float *)a.krot + (long long)(b * a.Hkv + hk) * a.Sk * D;  // raw keys
    const float *vh = (const float *)a.vt + (long long)(b * a.Hkv + hk) * a.Sk * D;
    // last key any query of this block may see (every key when not causal)
    const long long qpos_last = a.q_pos0 + min(a.Sq, qblk0 + 64) - 1;
    const long long kend_ll = a.causal ? min((long long)a.Sk, qpos_last - a.k_pos0 + 1) : (long long)a.Sk;
    const int kend = (int)max(0ll, kend_ll);

    float o[D];
#pragma unroll
    for (int c = 0; c < D; ++c) o[c] = 0.f;
    float m = -INFINITY, l = 0.f;
    unsigned long long skipped = 0;

    for (int j0 = 0; j0 < kend; j0 += TK) {
        __syncthreads();
        for (int e = lane; e < TK * P; e += 64) {
            const int jj = e / P, p = e % P, j = j0 + jj;
            float2 r = make_float2(0.f, 0.f);
            if (j < kend) {
                float c, s;
                rope_cos_sin(a.k_pos0 + j, a.theta[p], c, s);
                const int il = a.gptj ? 2 * p : p, ih = a.gptj ? 2 * p + 1 : p + P;
                const float x = kh[(long long)j * D + il], y = kh[(long long)j * D + ih];
                r = make_float2(x * c - y * s, y * c + x * s);
            }
            ks[jj][p] = r;
        }
        for (int e = lane; e < TK * D; e += 64) {
            const int jj = e / D, c = e % D, j = j0 + jj;
            vs[jj][c] = (j < kend) ? vh[(long long)j * D + c] : 0.f;
        }
        __syncthreads();
        const int nk = min(TK, kend - j0);
        for (int jj = 0; jj < nk; ++jj) {
            long long delta = qpos - (a.k_pos0 + j0 + jj);
            if (!valid || (a.causal && delta < 0)) continue;
            if (delta < 0) delta = -delta;  // windows on |i - j| when not causal
            float s = 0.f;
            int ndrop = 0;
#pragma unroll
            for (int p = 0; p < P; ++p) {
                const float term = qx[p] * ks[jj][p].x + qy[p] * ks[jj][p].y;
                const bool keep = delta <= (long long)a.W[p];
                s += keep ? term : 0.f;
                ndrop += keep ? 0 : 1;
            }
            skipped += (unsigned)ndrop;
            const float x = s * a.scale_log2;
            const float m_new = fmaxf(m, x);
            const float corr = exp2f(m - m_new);
            const float pe = exp2f(x - m_new);
            l = l * corr + pe;
#pragma unroll
            for (int c = 0; c < D; ++c) o[c] = o[c] * corr + pe * vs[jj][c];
            m = m_new;
        }
    }
    if (valid) {
        float *orow = (float *)a.out + ((long long)bh * a.Sq + i) * D;
        const float inv = 1.f / l;
#pragma unroll
        for (int c = 0; c < D; ++c) orow[c] = o[c] * inv;
    }
    skipped = wave_sum_u64(skipped);
    if (lane == 0 && skipped) atomicAdd(a.counter, skipped);
}

// ============================================================================
// Split-KV decode, bf16, on MFMA 16x16x32.  One workgroup = (split, b, kv
// head, slab of <= 8 query heads); its 4 waves take 32-key chunks of the
// split in turn (two groups of 16 keys).
//
// Scores S^T[16 keys x 16 head slots] per group: lane (t, q) = (lane % 16,
// lane / 16) owns key t of the group and rotates that key's pairs
// 16s + 4q + (0..3) of each K-step s.  A key at distance D keeps pairs
// [p*(D), P): the lane loads only the 8-byte pieces holding kept pairs (far
// keys read few bytes) and zeroes the dropped ones; K-steps no key of the
// chunk keeps are skipped.  cos/sin come from a two-level table (per-chunk
// coarse angle x per-key fine angle, both from fp64-reduced angles).
// The score output puts head t in lane column t, so each head's softmax
// statistics are in-lane plus a max over the 4 quads.
// P.V: O^T[16 dims x 16 heads] += V^T P^T.  The value chunk is staged in LDS
// by direct loads (issued right after the previous chunk's P.V, so they
// overlap this chunk's scores) and read back transposed with
// ds_read_b64_tr_b16, whose lane mapping (16-lane groups; output lane t,
// element c <- element t % 4 of the 8-byte read of source lane 4c + t / 4)
// yields dim t of 4 keys per read.  A combine kernel merges the splits.
// grid (nsplit, B*Hkv*n_slabs), block 256.
// ============================================================================


// 8 bytes holding dim t of 4 consecutive keys (see the lane mapping above)
__device__ inline u32x2 lds_read_tr16(const unsigned char *lds, unsigned byte_addr) {
    const s16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)(lds + byte_addr));
    return __builtin_bit_cast(u32x2, r);
}

// One 16-dim block of O^T += V^T P^T over a wave's chunk.  Two 16-key groups:
// MFMA 16x16x32, K index 8q + 4g + c = key 16g + 4q + c of the chunk (the
// probability words of both groups, and the value reads of both, side by
// side).  One group: MFMA 16x16x16 over keys 4q + c.
template <int NG>
__device__ inline f32x4_t decode_pv(const unsigned char *vb, unsigned addr0, unsigned addr1,
                                    const unsigned (&pw)[2 * NG], f32x4_t o) {
    const u32x2 v0 = lds_read_tr16(vb, addr0);
    if constexpr (NG == 2) {
        const u32x2 v1 = lds_read_tr16(vb, addr1);
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, (u32x4){v0.x, v0.y, v1.x, v1.y}),
                                                       __builtin_bit_cast(bf16x8_t, (u32x4){pw[0], pw[1], pw[2], pw[3]}),
                                                       o, 0, 0, 0);
    } else {
        (void)addr1;
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, v0),
                                                         __builtin_bit_cast(s16x4_t, (u32x2){pw[0], pw[1]}), o, 0, 0, 0);
    }
}

template <int D, bool GPTJ>
__global__ __launch_bounds__(256, D >= 256 ? 2 : 1) void decode_bf16_kernel(DecodeArgs a) {
    constexpr int P = D / 2;
    constexpr int NSTEP = D / 32;        // score K-steps of 16 pairs
    constexpr int NDB = D / 16;          // P.V output blocks of 16 dims
    constexpr int CK = (D >= 256) ? 16 : 32;  // keys per wave chunk (d = 256: half, for two workgroups per CU)
    constexpr int NG = CK / 16;          // 16-key groups per chunk
    constexpr int VROW = D * 2;          // bytes per value row
    constexpr int CHV = VROW / 16;       // 16-byte chunks per value row
    constexpr int VBYTES = CK * VROW;    // value chunk bytes (8 KB at d = 128 and 256)
    constexpr int VR = 1024 / VROW;      // value rows per 1 KB direct-load piece
    constexpr int H = kDecodeHeads;
    __shared__ float2 fine[P][CK];       // cos/sin(u * theta_p), u = 0..31
    __shared__ float2 coarse[4][P];      // per wave: cos/sin((pos0 + j0) * theta_p)
    __shared__ float2 stride_cs[P];      // cos/sin(4 * CK * theta_p): one wave step
    __shared__ __attribute__((aligned(1024))) unsigned char vbuf[4][VBYTES];
    __shared__ float wm[4][16], wl[4][16];

    const int split = blockIdx.x;
    const int slab = blockIdx.y % a.n_slabs;
    const int bk = blockIdx.y / a.n_slabs;
    const int b = bk / a.Hkv, hk = bk % a.Hkv;
    const int h0 = hk * a.group + slab * H;
    const int nh = min(H, a.group - slab * H);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int t = lane & 15, q = lane >> 4;

    for (int e = tid; e < P * CK; e += 256) {
        const int p = e / CK, u = e % CK;
        float c, s;
        rope_cos_sin(u, a.theta[p], c, s);
        fine[p][u] = make_float2(c, s);
    }
    if (tid < P) {
        float c, s;
        rope_cos_sin(4 * CK, a.theta[tid], c, s);
        stride_cs[tid] = make_float2(c, s);
    }
    const WaveWin<P> win = load_windows<P>(a.W);

    // query operand (B of the score MFMA): head slot t, pairs 16s + 4q + (0..3),
    // as decode_qrot_kernel rotated and scaled them; empty slots are 0
    bf16x8_t qf[NSTEP];
    {
        const unsigned *qrow = a.qrot + (long long)(b * a.Hq + h0 + t) * P;
#pragma unroll
        for (int s = 0; s < NSTEP; ++s) {
            u32x4 w = (u32x4){0u, 0u, 0u, 0u};
            if (t < nh) w = *(const u32x4 *)(qrow + 16 * s + 4 * q);
            qf[s] = __builtin_bit_cast(bf16x8_t, w);
        }
    }
    __syncthreads();

    const int ks = a.split_start[split];
    const int ke = min(a.split_start[split + 1], a.S);
    const unsigned short *kbase = (const unsigned short *)a.k + (long long)bk * a.S * D;
    const unsigned char *vbase = (const unsigned char *)a.v + (long long)bk * a.S * VROW;
    unsigned char *vb = vbuf[wave];

    // Value rows are staged with 16-byte chunks swizzled: row r, chunk c at
    // byte r*VROW + ((c ^ vsw(r)) << 4), vsw(r) = 2 (r mod CHV/2), so the
    // transposed reads of a 16-lane group (4 rows x 32 bytes) hit distinct
    // banks.  The chunk is prefetched into registers one chunk ahead (lane l
    // of 1 KB piece m holds LDS bytes 1024 m + 16 l: row VR m + l / CHV,
    // physical chunk l % CHV) and written to LDS when its turn comes.
    constexpr int NVP = VBYTES / 1024;  // pieces per chunk
    const int vlr = lane / CHV;
    auto vsw = [](int r) { return 2 * (r % (CHV / 2)); };
    u32x4 vreg[NVP];
#define DEC_LOAD_V(jc_)                                                                 \
    {                                                                                 \
        const int nrow_ = min(CK, ke - (jc_));  /* rows past the split repeat its last row */ \
        _Pragma("unroll") for (int m = 0; m < NVP; ++m) {                             \
            const int row_ = VR * m + vlr;                                            \
            const int c_ = (lane % CHV) ^ vsw(row_);                                  \
            const int grow_ = (jc_) + min(row_, nrow_ - 1);                           \
            vreg[m] = *(const u32x4 *)(vbase + (long long)grow_ * VROW + c_ * 16);    \
        }                                                                             \
    }
    // this lane's transposed-read byte address for output block db, key group hh
    auto vtr_addr = [&](int db, int hh) {
        const int row = 16 * hh + 4 * q + (t >> 2);
        const int col = 32 * db + 8 * (t & 3);  // byte column
        return (unsigned)(row * VROW + ((((col >> 4) ^ vsw(row)) << 4) | (col & 15)));
    };

    f32x4_t o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[db] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    constexpr float kRescale = 8.f;
    constexpr unsigned kOnesBf16x2 = 0x3f803f80u;
    float m_ref = 0.f, l_run = 0.f;
    bool first = true;
    unsigned long long skipped = 0;

    // Per-chunk key bookkeeping.  Dropped pairs per key: the chunk's nearest
    // key has the fewest (p_near, one ballot); farther keys add the few
    // windows that fall inside the chunk's distance range.
#define DEC_CHUNK_KEYS(jc_, smin_, ps0_, ps1_)                                          \
    {                                                                                 \
        const int d_near_ = a.S - min((jc_) + CK - 1, ke - 1);                        \
        const int d_far_ = a.S - (jc_);                                               \
        const int p_near_ = cut_below(win, d_near_);                                  \
        smin_ = p_near_ >> 4;                                                         \
        ps0_ = p_near_;                                                               \
        ps1_ = p_near_;                                                               \
        for (int pp = p_near_; pp < P - 1; ++pp) {                                    \
            const int wpp = window_at(win, pp);                                       \
            if (wpp >= d_far_) break;                                                 \
            ps0_ += (wpp < a.S - ((jc_) + t)) ? 1 : 0;                                \
            if (NG > 1) ps1_ += (wpp < a.S - ((jc_) + 16 + t)) ? 1 : 0;               \
        }                                                                             \
        if ((jc_) + t >= ke) ps0_ = P;                                                \
        if (NG > 1 && (jc_) + 16 + t >= ke) ps1_ = P;                                 \
    }
    // Key pieces of the last two K-steps (the only ones far keys keep) are
    // loaded one chunk ahead into registers; nearer steps load on use.  Every
    // load is issued unconditionally (fixed vmcnt bookkeeping, no divergent
    // branches): a piece the lane does not need reads the pieces of pairs
    // P-4..P-1 (never cut, so another lane fetches the same sectors anyway),
    // and the per-pair mask zeroes it.  In the interleaved layout a key's kept
    // pairs are one contiguous suffix of its row.
    constexpr int SPRE = (NSTEP >= 2) ? NSTEP - 2 : 0;
#define DEC_LOAD_K(jc_, ps0_, ps1_)                                                     \
    {                                                                                 \
        _Pragma("unroll") for (int g = 0; g < NG; ++g) {                              \
            const int psg_ = g ? (ps1_) : (ps0_);                                     \
            const unsigned short *kr_ = kbase + (long long)min((jc_) + 16 * g + t, ke - 1) * D; \
            _Pragma("unroll") for (int i = 0; i < NSTEP - SPRE; ++i) {                \
                const int pb_ = 16 * (SPRE + i) + 4 * q;                              \
                const int off_ = (pb_ + 4 > psg_) ? pb_ : (P - 4);                    \
                load_pair_pieces(kr_, off_, P, GPTJ, klo[g][i], khi[g][i]);            \
            }                                                                         \
        }                                                                             \
    }

    int j0 = ks + wave * CK;
    int s_min = 0, ps0 = P, ps1 = P;
    u32x2 klo[NG][NSTEP - SPRE], khi[NG][NSTEP - SPRE];
    if (j0 < ke) {
        DEC_LOAD_V(j0);
        DEC_CHUNK_KEYS(j0, s_min, ps0, ps1);
        DEC_LOAD_K(j0, ps0, ps1);
    }
    // coarse angle of this lane's pairs (lane, lane + 64, ...) at the wave's
    // current chunk start: exact every 16 chunks, advanced by one wave stride
    // in between
    constexpr int PPL = (P + 63) / 64;  // pairs per lane
    float2 cs_lane[PPL], cs_step[PPL];
#pragma unroll
    for (int e = 0; e < PPL; ++e) {
        cs_lane[e] = make_float2(1.f, 0.f);
        cs_step[e] = (lane + 64 * e < P) ? stride_cs[lane + 64 * e] : make_float2(1.f, 0.f);
    }
    for (int it = 0; j0 < ke; j0 += 4 * CK, ++it) {
        const int jn = j0 + 4 * CK;
        // this chunk's values to LDS (the previous chunk's transposed reads,
        // earlier in this wave's LDS order, are done with the buffer), then
        // the next chunk's values into the freed registers
#pragma unroll
        for (int m = 0; m < NVP; ++m) *(u32x4 *)(vb + m * 1024 + lane * 16) = vreg[m];
        if (jn < ke) DEC_LOAD_V(jn);
#pragma unroll
        for (int e = 0; e < PPL; ++e) {
            const int pl = lane + 64 * e;
            if (pl < P) {
                if ((it & 15) == 0) {
                    float c, s;
                    rope_cos_sin(a.pos0 + j0, a.theta[pl], c, s);
                    cs_lane[e] = make_float2(c, s);
                } else {
                    cs_lane[e] = make_float2(cs_lane[e].x * cs_step[e].x - cs_lane[e].y * cs_step[e].y,
                                             cs_lane[e].y * cs_step[e].x + cs_lane[e].x * cs_step[e].y);
                }
                coarse[wave][pl] = cs_lane[e];
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        f32x4_t sc[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const int u = 16 * g + t;  // key offset in the chunk
            const int ps = g ? ps1 : ps0;
            if (q == 0 && ps < P) skipped += (unsigned long long)ps * (unsigned)nh;
            const unsigned short *krow = kbase + (long long)min(j0 + u, ke - 1) * D;
            f32x4_t acc = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < NSTEP; ++s) {
                if (s < s_min) continue;
                const int pb = 16 * s + 4 * q;
                u32x2 lo, hi;
                if (s >= SPRE) {
                    lo = klo[g][s - SPRE];
                    hi = khi[g][s - SPRE];
                } else {
                    const int off = (pb + 4 > ps) ? pb : (P - 4);
                    load_pair_pieces(krow, off, P, GPTJ, lo, hi);
                }
                unsigned r[4];
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const int p = pb + w;
                    float x, y;
                    pair_xy(lo, hi, w, GPTJ, x, y);
                    const float2 f = fine[p][u];
                    const float2 cc = coarse[wave][p];
                    const float cs = f.x * cc.x - f.y * cc.y;
                    const float sn = f.y * cc.x + f.x * cc.y;
                    r[w] = (p < ps) ? 0u : pack_bf(x * cs - y * sn, y * cs + x * sn);
                }
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8_t, (u32x4){r[0], r[1], r[2], r[3]}), qf[s], acc, 0, 0, 0);
            }
            // rows of acc are keys 4q + (0..3) of the group; drop keys past the split
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (j0 + 16 * g + 4 * q + i >= ke) acc[i] = -INFINITY;
            sc[g] = acc;
        }

        // next chunk's keys: bookkeeping and the prefetched key pieces
        if (jn < ke) {
            DEC_CHUNK_KEYS(jn, s_min, ps0, ps1);
            DEC_LOAD_K(jn, ps0, ps1);
        }

        // online softmax per head slot t (log2 units, lazy reference)
        float bm = fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3]));
        if (NG > 1) bm = fmaxf(bm, fmaxf(fmaxf(sc[NG - 1][0], sc[NG - 1][1]), fmaxf(sc[NG - 1][2], sc[NG - 1][3])));
        bm = quad_max(bm);
        const bool move = first || bm > m_ref + kRescale;
        first = false;
        if (__ballot(move)) {
            const float m_new = move ? bm : m_ref;
            const float corr = fast_exp2(m_ref - m_new);
            m_ref = m_new;
            l_run *= corr;
#pragma unroll
            for (int db = 0; db < NDB; ++db) o[db] *= corr;
        }
        unsigned pw[2 * NG];
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            pw[2 * g] = pack_bf(fast_exp2(sc[g][0] - m_ref), fast_exp2(sc[g][1] - m_ref));
            pw[2 * g + 1] = pack_bf(fast_exp2(sc[g][2] - m_ref), fast_exp2(sc[g][3] - m_ref));
        }
#pragma unroll
        for (int i = 0; i < 2 * NG; ++i) l_run = dot2_bf(pw[i], kOnesBf16x2, l_run);

        // P.V on this chunk's values (written to LDS by this wave above)
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int db = 0; db < NDB; ++db) o[db] = decode_pv<NG>(vb, vtr_addr(db, 0), vtr_addr(db, NG - 1), pw, o[db]);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
#undef DEC_CHUNK_KEYS
#undef DEC_LOAD_K
#undef DEC_LOAD_V

    // ---- merge the 4 waves (reuses the value buffers) and write partials
    l_run = quad_sum(l_run);
    __syncthreads();
    float *wo = (float *)&vbuf[0][0];  // [4][H][D]
    if (t < nh) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i) wo[(wave * H + t) * D + 16 * db + 4 * q + i] = o[db][i];
    }
    if (q == 0) {
        wm[wave][t] = first ? -INFINITY : m_ref;  // a wave without keys contributes nothing
        wl[wave][t] = l_run;
    }
    __syncthreads();
    for (int e = tid; e < nh * (D + 2); e += 256) {
        const int hh = e / (D + 2), c = e % (D + 2);
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; ++w) M = fmaxf(M, wm[w][hh]);
        float val;
        if (c == D) {
            val = M;
        } else {
            val = 0.f;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float f = (wm[w][hh] == -INFINITY) ? 0.f : fast_exp2(wm[w][hh] - M);
                val += f * ((c < D) ? wo[(w * H + hh) * D + c] : wl[w][hh]);
            }
        }
        a.part[((long long)(b * a.Hq + h0 + hh) * a.nsplit + split) * (D + 2) + c] = val;
    }
    skipped = wave_sum_u64(skipped);
    if (lane == 0 && skipped) atomicAdd(a.counter, skipped);
}

// Ragged batch: sequence b gets a share of the split budget proportional to
// its length (at least 1, at most its 64-key chunks and the grid's width),
// so short sequences do not hold back long ones.  Every wave returns the same.
__device__ inline long long paged_total_len(const DecodeArgs &a) {
    const int lane = threadIdx.x & 63;
    unsigned long long tot = 0;
    for (int i = lane; i < a.B; i += 64) tot += (unsigned long long)min(max(a.seq_lens[i], 1), a.S);
    return (long long)wave_sum_u64(tot);
}
// Splits of sequence b: its share of `bud` splits, rounded up (so no split
// holds more than the batch's average share of keys), at least one.
__device__ inline int paged_nsplit_of(const DecodeArgs &a, int b, long long tot, long long bud) {
    const long long L = min(max(a.seq_lens[b], 1), a.S);
    const long long want = (L * bud + tot - 1) / tot;
    const long long nch = (L + kKeyTile - 1) / kKeyTile;
    return (int)max(1ll, min(want, min((long long)a.nsplit, nch)));
}
// The shares are taken of a budget lowered by the rounding excess until the
// batch's splits fit the workgroups resident at once (split_budget): one
// split more than that would run as a second wave and double the time.
// Every lane of the wave must call it (one sequence per lane, then a wave sum).
__device__ inline long long paged_budget(const DecodeArgs &a, long long tot) {
    const int lane = threadIdx.x & 63;
    long long bud = a.split_budget;
    for (int it = 0; it < 8; ++it) {
        unsigned long long part = 0;
        for (int i = lane; i < a.B; i += 64) part += (unsigned long long)paged_nsplit_of(a, i, tot, bud);
        const long long total = (long long)wave_sum_u64(part);
        if (total <= a.split_budget || bud <= 1) break;
        bud = max(1ll, bud - (total - a.split_budget));
    }
    return bud;
}
__device__ inline int paged_nsplit(const DecodeArgs &a, int b) {
    const long long tot = paged_total_len(a);
    return paged_nsplit_of(a, b, tot, paged_budget(a, tot));
}

// Algorithmic bytes of keys [0, j) of a sequence of S keys (decode query after
// them): 2d per value row plus 4 per kept pair, where pair p (finite W_p) is
// dropped for the keys j' < S - W_p, i.e. sum_p min(j, max(0, S - W_p))
// dropped pair-keys.  The windows are sorted, so with p1 = #{W_p <= S - j} and
// p2 = #{W_p < S} that sum is j p1 + sum_{p1 <= p < p2} (S - W_p): two ballot
// counts and a prefix table of the windows, no cross-lane sums.
template <int P>
struct WinPrefix {      // lane l: sum of the finite windows of pairs below l (and below 64 + l)
    long long lo, hi;
};
template <int P>
__device__ inline WinPrefix<P> win_prefix(const WaveWin<P> &win) {
    const int lane = threadIdx.x & 63;
    auto excl_scan = [&](int w) {
        const long long v = (w != kWindowInf) ? (long long)w : 0ll;
        long long incl = v;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const long long y = __shfl_up(incl, off, 64);
            if (lane >= off) incl += y;
        }
        return incl - v;
    };
    WinPrefix<P> r;
    r.lo = excl_scan(win.lo);
    r.hi = 0;
    if constexpr (P > 64) {
        const long long last = __shfl(r.lo, 63, 64) + (win.lo != kWindowInf ? (long long)__shfl(win.lo, 63, 64) : 0ll);
        r.hi = last + excl_scan(win.hi);
    }
    return r;
}
// sum of the finite windows of pairs [0, p), p wave-uniform
template <int P>
__device__ inline long long win_prefix_at(const WinPrefix<P> &pw, const WaveWin<P> &win, int p) {
    auto rl = [](long long v, int l) {
        const unsigned lo = __builtin_amdgcn_readlane((unsigned)v, l);
        const unsigned hi = __builtin_amdgcn_readlane((unsigned)((unsigned long long)v >> 32), l);
        return (long long)(((unsigned long long)hi << 32) | lo);
    };
    if (p < 64) return rl(pw.lo, p);
    if constexpr (P > 64) {
        if (p < 128) return rl(pw.hi, p - 64);
        const int w = __builtin_amdgcn_readlane(win.hi, 63);
        return rl(pw.hi, 63) + (w != kWindowInf ? (long long)w : 0ll);
    }
    const int w = __builtin_amdgcn_readlane(win.lo, 63);
    return rl(pw.lo, 63) + (w != kWindowInf ? (long long)w : 0ll);
}
template <int D>
__device__ inline long long dec_prefix_bytes(int j, int S, const WaveWin<D / 2> &win, const WinPrefix<D / 2> &pw) {
    constexpr int P = D / 2;
    const int p1 = cut_below(win, S - j + 1), p2 = cut_below(win, S);  // the infinite window never counts
    const long long dropped = (long long)j * p1 + (long long)(p2 - p1) * S -
                              (win_prefix_at<P>(pw, win, p2) - win_prefix_at<P>(pw, win, p1));
    return (long long)j * (2 * D + 4 * P) - 4 * dropped;
}

// ============================================================================
// Key-cache writer: rotates each key at its position and stores it in the
// plane layout described below (one thread per (key, 4-pair plane): 8 bytes
// of each rotary half in, 16 bytes out).  grid (x, B*Hkv), block 256.
// ============================================================================

template <int D>
__global__ __launch_bounds__(256) void kpack_bf16_kernel(KPackArgs a) {
    constexpr int P = D / 2, NPL = P / 4, CHV = D / 8;
    constexpr unsigned KPBLK = NPL * 1024;
    const int bk = blockIdx.y;
    // per token: NPL key planes, then (with values) CHV 16-byte value chunks
    const int U = a.v ? NPL + CHV : NPL;
    const long long total = (long long)a.n * U;
    for (long long e = (long long)blockIdx.x * 256 + threadIdx.x; e < total; e += (long long)gridDim.x * 256) {
        const int i = (int)(e / U), pg = (int)(e % U);
        const long long j = a.k_begin + i;
        if (pg >= NPL) {  // value row j, chunk pg - NPL
            const int c = pg - NPL;
            const u32x4 val = *(const u32x4 *)((const unsigned short *)a.v + ((long long)bk * a.n + i) * D + c * 8);
            *(u32x4 *)((unsigned short *)a.vc + ((long long)bk * a.cap + j) * D + c * 8) = val;
            continue;
        }
        const unsigned short *src = (const unsigned short *)a.k + ((long long)bk * a.n + i) * D;
        u32x2 lo, hi;
        load_pair_pieces(src, 4 * pg, P, a.gptj != 0, lo, hi);
        unsigned r[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            float x, y, c, sn;
            pair_xy(lo, hi, w, a.gptj != 0, x, y);
            rope_cos_sin(a.pos0 + j, a.theta[4 * pg + w], c, sn);
            r[w] = pack_bf(x * c - y * sn, y * c + x * sn);
        }
        unsigned char *dst = (unsigned char *)a.kc +
                             ((long long)bk * (a.cap / kKeyTile) + j / kKeyTile) * KPBLK + pg * 1024 + (j % kKeyTile) * 16;
        *(u32x4 *)dst = (u32x4){r[0], r[1], r[2], r[3]};
    }
}

// ============================================================================
// Paged cache writer: token i of each sequence goes to the page holding its
// 64-key block; keys rotated into the plane layout (as kpack_bf16_kernel),
// values copied as rows.  One thread per (token, 16-byte unit).
// grid (x, B*Hkv), block 256.
// ============================================================================

template <int D>
__global__ __launch_bounds__(256) void paged_write_bf16_kernel(PagedWriteArgs a) {
    constexpr int P = D / 2, NPL = P / 4, CHV = D / 8, U = NPL + CHV;
    constexpr unsigned KPBLK = NPL * 1024;
    const int bk = blockIdx.y, b = bk / a.Hkv, hk = bk % a.Hkv;
    const long long total = (long long)a.n * U;
    for (long long e = (long long)blockIdx.x * 256 + threadIdx.x; e < total; e += (long long)gridDim.x * 256) {
        const int i = (int)(e / U), u = (int)(e % U);
        const long long j = a.k_begin + i;
        int page = a.page_table[(long long)b * a.max_pages + (int)(j / kKeyTile)];
        page = min(max(page, 0), a.num_pages - 1);
        const long long blk = (long long)page * a.Hkv + hk;
        const long long src_row = ((long long)bk * a.n + i) * D;
        if (u < NPL) {
            const unsigned short *src = (const unsigned short *)a.k + src_row;
            u32x2 lo, hi;
            load_pair_pieces(src, 4 * u, P, a.gptj != 0, lo, hi);
            unsigned r[4];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                float x, y, c, sn;
                pair_xy(lo, hi, w, a.gptj != 0, x, y);
                rope_cos_sin(a.pos0 + j, a.theta[4 * u + w], c, sn);
                r[w] = pack_bf(x * c - y * sn, y * c + x * sn);
            }
            *(u32x4 *)((unsigned char *)a.kpool + blk * KPBLK + u * 1024 + (j % kKeyTile) * 16) =
                (u32x4){r[0], r[1], r[2], r[3]};
        } else {
            const int c = u - NPL;
            *(u32x4 *)((unsigned char *)a.vpool + blk * (kKeyTile * D * 2) + (j % kKeyTile) * (D * 2) + c * 16) =
                *(const u32x4 *)((const unsigned short *)a.v + src_row + 8 * c);
        }
    }
}

// ============================================================================
// Split-KV decode over a key cache laid out for the windows (bf16).  Keys are
// stored rotated (at their own positions) in 64-key blocks of P/4 planes; plane
// pg holds pairs 4pg .. 4pg+3 of the block's 64 keys, 16 bytes per key, word w
// = (x'_p, y'_p) of pair p = 4pg + w:
//     byte ((b*Hkv + h) * cap/64 + j/64) * (P/4 * 1024) + pg * 1024 + (j % 64) * 16.
// A key at distance D keeps pairs [p*(D), P), so a block keeps a suffix of its
// planes, one contiguous byte range: the planes below the nearest key's cut
// are never read, and HBM traffic shrinks with distance (in the standard
// [S][d] layout each rotary half of a key is one 128-byte line that always
// holds kept pairs, so every line is read).  The plane's 16 bytes are the
// score MFMA's key operand as they stand: no rotation work in the loop.
// Values stay in the standard layout, row stride cap.  Same split, chunk,
// softmax, P.V and merge scheme as decode_bf16_kernel.
// grid (nsplit, B*Hkv*n_slabs), block 256.
// ============================================================================

template <int D, bool PAGED>
__global__ __launch_bounds__(256, D >= 256 ? 2 : 1) void decode_kcache_bf16_kernel(DecodeArgs a) {
    constexpr int P = D / 2;
    constexpr int NSTEP = D / 32;        // score K-steps of 16 pairs
    constexpr int NDB = D / 16;          // P.V output blocks of 16 dims
    constexpr int CK = (D >= 256) ? 16 : 32;  // keys per wave chunk (d = 256: half, for two workgroups per CU)
    constexpr int NG = CK / 16;          // 16-key groups per chunk
    constexpr int VROW = D * 2;          // bytes per value row
    constexpr int CHV = VROW / 16;       // 16-byte chunks per value row
    constexpr int VBYTES = CK * VROW;    // value chunk bytes (8 KB at d = 128 and 256)
    constexpr int VR = 1024 / VROW;      // value rows per 1 KB direct-load piece
    constexpr int H = kDecodeHeads;
    constexpr unsigned KPBLK = (P / 4) * 1024;  // bytes of one 64-key block of the key cache
    __shared__ __attribute__((aligned(1024))) unsigned char vbuf[4][VBYTES];
    __shared__ float wm[4][16], wl[4][16];

    // work item.  Paged: blockIdx.x walks the batch's splits (sequence b owns
    // nsb_b consecutive ids); blockIdx.y is (kv head, slab).  Otherwise
    // blockIdx.x is the split and blockIdx.y is (b, kv head, slab).
    int split = blockIdx.x, b, hk, nsb = 0;
    const int slab = blockIdx.y % a.n_slabs;
    if (PAGED) {
        hk = blockIdx.y / a.n_slabs;
        const long long tot = paged_total_len(a);
        const long long bud = paged_budget(a, tot);
        // the sequence owning split id `split`: 64 sequences per step, one per
        // lane, with a wave prefix sum of their split counts
        b = -1;
        const int lane_ = threadIdx.x & 63;
        for (int base_i = 0, c0 = 0; base_i < a.B; base_i += 64) {
            const int i = base_i + lane_;
            const int n = i < a.B ? paged_nsplit_of(a, i, tot, bud) : 0;
            int incl = n;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int y = __shfl_up(incl, off, 64);
                if (lane_ >= off) incl += y;
            }
            const int chunk = __shfl(incl, 63, 64);
            if (split < c0 + chunk) {
                const int first = __builtin_ctzll(__ballot(split < c0 + incl));
                const int excl = __shfl(incl - n, first, 64);
                nsb = __shfl(n, first, 64);
                b = base_i + first;
                split -= c0 + excl;
                break;
            }
            c0 += chunk;
        }
        if (b < 0) return;  // past the batch's splits (uniform)
    } else {
        const int bk0 = blockIdx.y / a.n_slabs;
        b = bk0 / a.Hkv;
        hk = bk0 % a.Hkv;
    }
    const int bk = b * a.Hkv + hk;
    const int h0 = hk * a.group + slab * H;
    const int nh = min(H, a.group - slab * H);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int t = lane & 15, q = lane >> 4;
    // keys of this sequence (ragged when paged: clamped to [1, a.S], a.S = max_len)
    const int S = PAGED ? min(max(a.seq_lens[b], 1), a.S) : a.S;

    const WaveWin<P> win = load_windows<P>(a.W);

    // query operand (B of the score MFMA): head slot t, pairs 16s + 4q + (0..3),
    // as decode_qrot_kernel rotated and scaled them; empty slots are 0
    bf16x8_t qf[NSTEP];
    {
        const unsigned *qrow = a.qrot + (long long)(b * a.Hq + h0 + t) * P;
#pragma unroll
        for (int s = 0; s < NSTEP; ++s) {
            u32x4 w = (u32x4){0u, 0u, 0u, 0u};
            if (t < nh) w = *(const u32x4 *)(qrow + 16 * s + 4 * q);
            qf[s] = __builtin_bit_cast(bf16x8_t, w);
        }
    }
    __syncthreads();

    int ks, ke;
    if (PAGED) {
        // byte-balanced split boundaries of this sequence (same rule as the host
        // planner): split s of nsb starts at the first 64-key chunk whose
        // prefix of algorithmic bytes reaches s / nsb of the total; splits past
        // nsb have no keys
        const WinPrefix<P> pw = win_prefix<P>(win);
        const long long total = dec_prefix_bytes<D>(S, S, win, pw);
        const int nchunks = (S + kKeyTile - 1) / kKeyTile;
        auto start_of = [&](int sp) {
            const long long target = total * min(sp, nsb) / nsb;
            int lo = 0, hi = nchunks;
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (dec_prefix_bytes<D>(min(S, mid * kKeyTile), S, win, pw) < target) lo = mid + 1; else hi = mid;
            }
            return lo * kKeyTile;
        };
        ks = start_of(split);
        ke = min(start_of(split + 1), S);
    } else {
        ks = a.split_start[split];
        ke = min(a.split_start[split + 1], S);
    }
    // key block c (64 keys) and its value rows
    auto page_of = [&](int c) {
        return min(max(a.page_table[(long long)b * a.max_pages + c], 0), a.num_pages - 1);
    };
    // block slot of key block c in the key / value arrays; when paged, each
    // chunk's slot is looked up two chunks ahead so the table read is off the
    // load path
    auto slot_of = [&](int c) -> long long {
        return PAGED ? ((long long)page_of(c) * a.Hkv + hk) : ((long long)bk * (a.cap / kKeyTile) + c);
    };
    auto kblock = [&](long long sl) { return (const unsigned char *)a.k + sl * KPBLK; };
    auto vblock = [&](long long sl) { return (const unsigned char *)a.v + sl * (kKeyTile * VROW); };
    unsigned char *vb = vbuf[wave];

    // Value rows are staged with 16-byte chunks swizzled: row r, chunk c at
    // byte r*VROW + ((c ^ vsw(r)) << 4), vsw(r) = 2 (r mod CHV/2), so the
    // transposed reads of a 16-lane group (4 rows x 32 bytes) hit distinct
    // banks.  The chunk is prefetched into registers one chunk ahead (lane l
    // of 1 KB piece m holds LDS bytes 1024 m + 16 l: row VR m + l / CHV,
    // physical chunk l % CHV) and written to LDS when its turn comes.
    constexpr int NVP = VBYTES / 1024;  // pieces per chunk
    const int vlr = lane / CHV;
    auto vsw = [](int r) { return 2 * (r % (CHV / 2)); };
    u32x4 vreg[NVP];
#define DEC_LOAD_V(jc_, sl_)                                                            \
    {                                                                                 \
        const int nrow_ = min(CK, ke - (jc_));  /* rows past the split repeat its last row */ \
        const unsigned char *vb_ = vblock(sl_);                                       \
        _Pragma("unroll") for (int m = 0; m < NVP; ++m) {                             \
            const int row_ = VR * m + vlr;                                            \
            const int c_ = (lane % CHV) ^ vsw(row_);                                  \
            const int brow_ = (jc_) % kKeyTile + min(row_, nrow_ - 1);                \
            vreg[m] = *(const u32x4 *)(vb_ + brow_ * VROW + c_ * 16);                 \
        }                                                                             \
    }
    // this lane's transposed-read byte address for output block db, key group hh
    auto vtr_addr = [&](int db, int hh) {
        const int row = 16 * hh + 4 * q + (t >> 2);
        const int col = 32 * db + 8 * (t & 3);  // byte column
        return (unsigned)(row * VROW + ((((col >> 4) ^ vsw(row)) << 4) | (col & 15)));
    };

    f32x4_t o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[db] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    constexpr float kRescale = 8.f;
    constexpr unsigned kOnesBf16x2 = 0x3f803f80u;
    float m_ref = 0.f, l_run = 0.f;
    bool first = true;
    unsigned long long skipped = 0;

    // Per-chunk key bookkeeping.  Dropped pairs per key: the chunk's nearest
    // key has the fewest (p_near, one ballot); farther keys add the few
    // windows that fall inside the chunk's distance range.
#define DEC_CHUNK_KEYS(jc_, smin_, ps0_, ps1_)                                          \
    {                                                                                 \
        const int d_near_ = S - min((jc_) + CK - 1, ke - 1);                          \
        const int d_far_ = S - (jc_);                                                 \
        const int p_near_ = cut_below(win, d_near_);                                  \
        smin_ = p_near_ >> 4;                                                         \
        pmin = p_near_ >> 2;                                                          \
        ps0_ = p_near_;                                                               \
        ps1_ = p_near_;                                                               \
        for (int pp = p_near_; pp < P - 1; ++pp) {                                    \
            const int wpp = window_at(win, pp);                                       \
            if (wpp >= d_far_) break;                                                 \
            ps0_ += (wpp < S - ((jc_) + t)) ? 1 : 0;                                  \
            if (NG > 1) ps1_ += (wpp < S - ((jc_) + 16 + t)) ? 1 : 0;                 \
        }                                                                             \
        if ((jc_) + t >= ke) ps0_ = P;                                                \
        if (NG > 1 && (jc_) + 16 + t >= ke) ps1_ = P;                                 \
    }
    // Key planes of the last two K-steps (the only ones far keys keep) are
    // loaded one chunk ahead into registers; nearer steps load on use.  A lane
    // whose plane (4 s + q) lies wholly below the chunk's nearest key's cut
    // reads past the end of the block's buffer: zeros, and no memory traffic.
    // Rows past the split repeat its last key.
    constexpr int SPRE = (NSTEP >= 2) ? NSTEP - 2 : 0;
#define DEC_KOFF(pg_, row_) (((pg_) >= pmin) ? (unsigned)((pg_) * 1024 + (row_) * 16) : KPBLK)
#define DEC_LOAD_K(jc_, sl_)                                                            \
    {                                                                                 \
        const __amdgpu_buffer_rsrc_t kr_ = raw_rsrc(kblock(sl_), KPBLK);              \
        _Pragma("unroll") for (int g = 0; g < NG; ++g) {                              \
            const int row_ = min((jc_) + 16 * g + t, ke - 1) % kKeyTile;               \
            _Pragma("unroll") for (int i = 0; i < NSTEP - SPRE; ++i)                  \
                kreg[g][i] = raw_load16(kr_, DEC_KOFF(4 * (SPRE + i) + q, row_));     \
        }                                                                             \
    }

    int j0 = ks + wave * CK;
    int s_min = 0, ps0 = P, ps1 = P, pmin = 0;
    u32x4 kreg[NG][NSTEP - SPRE];
    long long sl_cur = 0, sl_nxt = 0;
    if (j0 < ke) {
        sl_cur = slot_of(j0 / kKeyTile);
        if (j0 + 4 * CK < ke) sl_nxt = slot_of((j0 + 4 * CK) / kKeyTile);
        DEC_LOAD_V(j0, sl_cur);
        DEC_CHUNK_KEYS(j0, s_min, ps0, ps1);
        DEC_LOAD_K(j0, sl_cur);
    }
    for (; j0 < ke; j0 += 4 * CK) {
        const int jn = j0 + 4 * CK;
        const long long sl_nn = (jn + 4 * CK < ke) ? slot_of((jn + 4 * CK) / kKeyTile) : 0;
        // this chunk's values to LDS (the previous chunk's transposed reads,
        // earlier in this wave's LDS order, are done with the buffer), then
        // the next chunk's values into the freed registers
#pragma unroll
        for (int m = 0; m < NVP; ++m) *(u32x4 *)(vb + m * 1024 + lane * 16) = vreg[m];
        if (jn < ke) DEC_LOAD_V(jn, sl_nxt);
        const __amdgpu_buffer_rsrc_t kr = raw_rsrc(kblock(sl_cur), KPBLK);

        f32x4_t sc[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const int u = 16 * g + t;  // key offset in the chunk
            const int ps = g ? ps1 : ps0;
            if (q == 0 && ps < P) skipped += (unsigned long long)ps * (unsigned)nh;
            const int row = min(j0 + u, ke - 1) % kKeyTile;
            f32x4_t acc = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < NSTEP; ++s) {
                if (s < s_min) continue;
                const int pb = 16 * s + 4 * q;
                const u32x4 kw = (s >= SPRE) ? kreg[g][s - SPRE] : raw_load16(kr, DEC_KOFF(4 * s + q, row));
                // words are rotated pairs (x'_p, y'_p), p = pb + w; drop p < p*(key)
                const u32x4 r = (u32x4){(pb + 0 < ps) ? 0u : kw.x, (pb + 1 < ps) ? 0u : kw.y,
                                        (pb + 2 < ps) ? 0u : kw.z, (pb + 3 < ps) ? 0u : kw.w};
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, r), qf[s], acc, 0, 0, 0);
            }
            // rows of acc are keys 4q + (0..3) of the group; drop keys past the split
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (j0 + 16 * g + 4 * q + i >= ke) acc[i] = -INFINITY;
            sc[g] = acc;
        }

        // next chunk's keys: bookkeeping and the prefetched key pieces
        if (jn < ke) {
            DEC_CHUNK_KEYS(jn, s_min, ps0, ps1);
            DEC_LOAD_K(jn, sl_nxt);
        }

        // online softmax per head slot t (log2 units, lazy reference)
        float bm = fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3]));
        if (NG > 1) bm = fmaxf(bm, fmaxf(fmaxf(sc[NG - 1][0], sc[NG - 1][1]), fmaxf(sc[NG - 1][2], sc[NG - 1][3])));
        bm = quad_max(bm);
        const bool move = first || bm > m_ref + kRescale;
        first = false;
        if (__ballot(move)) {
            const float m_new = move ? bm : m_ref;
            const float corr = fast_exp2(m_ref - m_new);
            m_ref = m_new;
            l_run *= corr;
#pragma unroll
            for (int db = 0; db < NDB; ++db) o[db] *= corr;
        }
        unsigned pw[2 * NG];
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            pw[2 * g] = pack_bf(fast_exp2(sc[g][0] - m_ref), fast_exp2(sc[g][1] - m_ref));
            pw[2 * g + 1] = pack_bf(fast_exp2(sc[g][2] - m_ref), fast_exp2(sc[g][3] - m_ref));
        }
#pragma unroll
        for (int i = 0; i < 2 * NG; ++i) l_run = dot2_bf(pw[i], kOnesBf16x2, l_run);

        // P.V on this chunk's values (written to LDS by this wave above)
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int db = 0; db < NDB; ++db) o[db] = decode_pv<NG>(vb, vtr_addr(db, 0), vtr_addr(db, NG - 1), pw, o[db]);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        sl_cur = sl_nxt;
        sl_nxt = sl_nn;
    }
#undef DEC_CHUNK_KEYS
#undef DEC_LOAD_K
#undef DEC_LOAD_V
#undef DEC_KOFF

    // ---- merge the 4 waves (reuses the value buffers) and write partials
    l_run = quad_sum(l_run);
    __syncthreads();
    float *wo = (float *)&vbuf[0][0];  // [4][H][D]
    if (t < nh) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i) wo[(wave * H + t) * D + 16 * db + 4 * q + i] = o[db][i];
    }
    if (q == 0) {
        wm[wave][t] = first ? -INFINITY : m_ref;  // a wave without keys contributes nothing
        wl[wave][t] = l_run;
    }
    __syncthreads();
    for (int e = tid; e < nh * (D + 2); e += 256) {
        const int hh = e / (D + 2), c = e % (D + 2);
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; ++w) M = fmaxf(M, wm[w][hh]);
        float val;
        if (c == D) {
            val = M;
        } else {
            val = 0.f;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float f = (wm[w][hh] == -INFINITY) ? 0.f : fast_exp2(wm[w][hh] - M);
                val += f * ((c < D) ? wo[(w * H + hh) * D + c] : wl[w][hh]);
            }
        }
        a.part[((long long)(b * a.Hq + h0 + hh) * a.nsplit + split) * (D + 2) + c] = val;
    }
    skipped = wave_sum_u64(skipped);
    if (lane == 0 && skipped) atomicAdd(a.counter, skipped);
}


// Merge the ns split partials of one row (pr[s * (D + 2) + ...] = o..., m, l):
// out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s, for dim c.  Splits are
// read CU at a time (indices clamped to the row's last split, extra values
// masked), so CU loads are in flight per step; the sum runs in split order.
template <int D>
__device__ inline float combine_row(const float *pr, int ns, int c) {
    constexpr int CU = 8;
    float M = -INFINITY;
    for (int s0 = 0; s0 < ns; s0 += CU) {
        float m[CU];
#pragma unroll
        for (int u = 0; u < CU; ++u) m[u] = pr[min(s0 + u, ns - 1) * (D + 2) + D];
#pragma unroll
        for (int u = 0; u < CU; ++u) M = fmaxf(M, m[u]);  // a repeated last split changes no max
    }
    float num = 0.f, den = 0.f;
    for (int s0 = 0; s0 < ns; s0 += CU) {
        float m[CU], o[CU], l[CU];
#pragma unroll
        for (int u = 0; u < CU; ++u) {
            const float *ps = pr + min(s0 + u, ns - 1) * (D + 2);
            m[u] = ps[D];
            o[u] = ps[c];
            l[u] = ps[D + 1];
        }
#pragma unroll
        for (int u = 0; u < CU; ++u) {
            if (s0 + u >= ns || m[u] == -INFINITY) continue;
            const float f = fast_exp2(m[u] - M);
            num += f * o[u];
            den += f * l[u];
        }
    }
    return num / den;
}

// Decode: grid B*Hq, block D.
template <int D, bool PAGED>
__global__ __launch_bounds__(D) void decode_combine_kernel(DecodeArgs a) {
    const int row = blockIdx.x, c = threadIdx.x;
    const float *pr = a.part + (long long)row * a.nsplit * (D + 2);
    const int ns = PAGED ? paged_nsplit(a, row / a.Hq) : a.nsplit;
    ((__bf16 *)a.out)[(long long)row * D + c] = (__bf16)combine_row<D>(pr, ns, c);
}

// Merge of a key-split prefill: grid B*Hq*Sq (one query row each), block D,
// one thread per dim walking every split (few splits: chunks of many
// queries).
template <int D>
__global__ __launch_bounds__(D) void prefill_combine_kernel(AttnArgs a) {
    const long long row = blockIdx.x;
    const int c = threadIdx.x;
    const float *pr = a.part + row * a.n_ksplit * (D + 2);
    ((__bf16 *)a.out)[row * D + c] = (__bf16)combine_row<D>(pr, a.n_ksplit, c);
}

// The same merge with many splits: grid B*Hq*Sq, block kCombineGroups * D.
// Each group of D threads merges every kCombineGroups-th split of dim c with
// a running maximum (one pass over the partials, four loads in flight per
// thread), then the groups' (max, numerator, denominator) meet in LDS.  Many
// splits and few rows (a short chunk: 64 splits, 448 rows) keep more loads in
// flight this way than one thread per dim walking all splits twice.
constexpr int kCombineGroups = 4;
template <int D>
__global__ __launch_bounds__(D * kCombineGroups) void prefill_combine_wide_kernel(AttnArgs a) {
    constexpr int G = kCombineGroups, U = 4;
    __shared__ float red[3][G][D];
    const long long row = blockIdx.x;
    const int c = threadIdx.x % D, gr = threadIdx.x / D;
    const int ns = a.n_ksplit;
    const float *pr = a.part + row * ns * (D + 2);
    float M = -INFINITY, num = 0.f, den = 0.f;
    for (int s0 = gr; s0 < ns; s0 += G * U) {
        float m[U], o[U], l[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int s = s0 + u * G;
            m[u] = -INFINITY;
            o[u] = l[u] = 0.f;
            if (s < ns) {
                const float *ps = pr + s * (D + 2);
                m[u] = ps[D];
                o[u] = ps[c];
                l[u] = ps[D + 1];
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (m[u] == -INFINITY) continue;  // a split with none of the row's mass (or past the end)
            if (m[u] > M) {
                const float r = fast_exp2(M - m[u]);  // 0 while M is -inf
                num *= r;
                den *= r;
                M = m[u];
            }
            const float f = fast_exp2(m[u] - M);
            num += f * o[u];
            den += f * l[u];
        }
    }
    red[0][gr][c] = M;
    red[1][gr][c] = num;
    red[2][gr][c] = den;
    __syncthreads();
    if (gr == 0) {
        float Mt = red[0][0][c];
#pragma unroll
        for (int g = 1; g < G; ++g) Mt = fmaxf(Mt, red[0][g][c]);
        float nt = 0.f, dt = 0.f;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const float mg = red[0][g][c];
            if (mg == -INFINITY) continue;
            const float f = fast_exp2(mg - Mt);
            nt += f * red[1][g][c];
            dt += f * red[2][g][c];
        }
        ((__bf16 *)a.out)[row * D + c] = (__bf16)(nt / dt);
    }
}

__global__ void fill_zero_u64_kernel(unsigned long long *p) { *p = 0ull; }

// Each query row rotated and pre-scaled once, as the pair words of the
// 16x16x32 kernel's query operand (pair p: (x'_p, y'_p) * log2(e)/sqrt(d) as
// bf16, x' in the low half), so the key-split workgroups of a short chunk
// load them instead of each rotating them again; also clears the counter.
// grid B*Hq*Sq rows, block d/2 (one pair per thread).
template <int D>
__global__ __launch_bounds__(D / 2) void prefill_qrot_kernel(AttnArgs a) {
    constexpr int P = D / 2;
    const long long row = blockIdx.x;
    const int i = (int)(row % a.Sq), p = threadIdx.x;
    if (row == 0 && p == 0) *a.counter = 0ull;
    const unsigned short *qrow = (const unsigned short *)a.q + row * D;
    float x, y;
    if (a.gptj) {
        const unsigned w = ((const unsigned *)qrow)[p];
        x = bf_lo(w);
        y = bf_hi(w);
    } else {
        x = __uint_as_float((unsigned)qrow[p] << 16);
        y = __uint_as_float((unsigned)qrow[p + P] << 16);
    }
    float c, sn;
    rope_cos_sin(a.q_pos0 + i, a.theta[p], c, sn);
    const float sc = a.scale_log2;
    a.qrot[row * P + p] = pack_bf((x * c - y * sn) * sc, (y * c + x * sn) * sc);
}

// The decode queries, rotated once per call at their position (pos0 + S, or
// pos0 + seq_lens[b] when paged) and scaled by log2(e)/sqrt(d): word p of row
// b*Hq + h is (x'_p, x'_{p+P}) in bf16, the score MFMA's operand order, so the
// split kernels load their query operand instead of each rotating it.  Also
// clears the dropped-term counter.  grid B*Hq, block P.
template <int D, bool PAGED>
__global__ __launch_bounds__(D / 2) void decode_qrot_kernel(DecodeArgs a) {
    constexpr int P = D / 2;
    const int row = blockIdx.x, p = threadIdx.x;
    if (row == 0 && p == 0) *a.counter = 0ull;
    const int b = row / a.Hq;
    const int S = PAGED ? min(max(a.seq_lens[b], 1), a.S) : a.S;
    const unsigned short *qrow = (const unsigned short *)a.q + (long long)row * D;
    const int ix = a.gptj ? 2 * p : p, iy = a.gptj ? 2 * p + 1 : p + P;
    const float x = __uint_as_float((unsigned)qrow[ix] << 16), y = __uint_as_float((unsigned)qrow[iy] << 16);
    float c, sn;
    rope_cos_sin(a.pos0 + S, a.theta[p], c, sn);
    a.qrot[(long long)row * P + p] = pack_bf((x * c - y * sn) * a.scale_log2, (y * c + x * sn) * a.scale_log2);
}

template <bool PAGED>
void launch_decode_qrot(const DecodeArgs &a, int d, hipStream_t s) {
    const unsigned rows = (unsigned)(a.B * a.Hq);
    if (d == 256) decode_qrot_kernel<256, PAGED><<<rows, 128, 0, s>>>(a);
    else if (d == 128) decode_qrot_kernel<128, PAGED><<<rows, 64, 0, s>>>(a);
    else decode_qrot_kernel<64, PAGED><<<rows, 32, 0, s>>>(a);
}

}  // namespace

// ---------------------------------------------------------------- launchers

hipError_t launch_prep_bf16(const PrepArgs &a, int d, hipStream_t s) {
    // one block per (tile, b x kv head, 16 pairs): an append of a few keys
    // rotates them across d / 32 blocks instead of one
    dim3 grid((unsigned)a.n_tiles, (unsigned)(a.B * a.Hkv), (unsigned)(d / 32));
    if (d == 256) prep_bf16_kernel<256><<<grid, 256, 0, s>>>(a);
    else if (d == 128) prep_bf16_kernel<128><<<grid, 256, 0, s>>>(a);
    else prep_bf16_kernel<64><<<grid, 256, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_prep_f32(const PrepArgs &a, int, hipStream_t s) {
    fill_zero_u64_kernel<<<1, 1, 0, s>>>(a.counter);
    return hipGetLastError();
}

hipError_t launch_prefill_bf16(const AttnArgs &a, int d, hipStream_t s) {
    // one workgroup per (work item, key split, head or slab), dealt to XCDs
    const dim3 grid((unsigned)(((a.n_groups * a.n_ksplit + 7) / 8) * 8 * a.group));
    if (d == 256) {
        if (a.causal) prefill16_bf16_kernel<256, true><<<grid, kPrefill16Waves * 64, 0, s>>>(a);
        else prefill16_bf16_kernel<256, false><<<grid, kPrefill16Waves * 64, 0, s>>>(a);
    } else if (a.narrow) {  // d = 128, at most 16 queries: 16-query waves
        if (a.causal) prefill16_bf16_kernel<128, true><<<grid, kPrefill16Waves * 64, 0, s>>>(a);
        else prefill16_bf16_kernel<128, false><<<grid, kPrefill16Waves * 64, 0, s>>>(a);
    } else if (a.causal) {
        if (d == 128) prefill_bf16_kernel<128, true><<<grid, kPrefillWaves * 64, 0, s>>>(a);
        else prefill_bf16_kernel<64, true><<<grid, kPrefillWaves * 64, 0, s>>>(a);
    } else {
        if (d == 128) prefill_bf16_kernel<128, false><<<grid, kPrefillWaves * 64, 0, s>>>(a);
        else prefill_bf16_kernel<64, false><<<grid, kPrefillWaves * 64, 0, s>>>(a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.n_ksplit <= 1) return e;
    const unsigned rows = (unsigned)((long long)a.B * a.Hq * a.Sq);
    if (a.n_ksplit >= 4 * kCombineGroups) {
        if (d == 256) prefill_combine_wide_kernel<256><<<rows, 256 * kCombineGroups, 0, s>>>(a);
        else if (d == 128) prefill_combine_wide_kernel<128><<<rows, 128 * kCombineGroups, 0, s>>>(a);
        else prefill_combine_wide_kernel<64><<<rows, 64 * kCombineGroups, 0, s>>>(a);
    } else {
        if (d == 256) prefill_combine_kernel<256><<<rows, 256, 0, s>>>(a);
        else if (d == 128) prefill_combine_kernel<128><<<rows, 128, 0, s>>>(a);
        else prefill_combine_kernel<64><<<rows, 64, 0, s>>>(a);
    }
    return hipGetLastError();
}

hipError_t launch_attend_f32(const AttnArgs &a, int d, hipStream_t s) {
    dim3 grid((unsigned)((a.Sq + 63) / 64), (unsigned)(a.B * a.Hq));
    if (d == 256) attend_f32_kernel<256><<<grid, 64, 0, s>>>(a);
    else if (d == 128) attend_f32_kernel<128><<<grid, 64, 0, s>>>(a);
    else attend_f32_kernel<64><<<grid, 64, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_decode_bf16(const DecodeArgs &a, int d, hipStream_t s) {
    launch_decode_qrot<false>(a, d, s);
    dim3 grid((unsigned)a.nsplit, (unsigned)(a.B * a.Hkv * a.n_slabs));
    if (d == 256 && a.gptj) decode_bf16_kernel<256, true><<<grid, 256, 0, s>>>(a);
    else if (d == 256) decode_bf16_kernel<256, false><<<grid, 256, 0, s>>>(a);
    else if (d == 128 && a.gptj) decode_bf16_kernel<128, true><<<grid, 256, 0, s>>>(a);
    else if (d == 128) decode_bf16_kernel<128, false><<<grid, 256, 0, s>>>(a);
    else if (a.gptj) decode_bf16_kernel<64, true><<<grid, 256, 0, s>>>(a);
    else decode_bf16_kernel<64, false><<<grid, 256, 0, s>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (d == 256) decode_combine_kernel<256, false><<<a.B * a.Hq, 256, 0, s>>>(a);
    else if (d == 128) decode_combine_kernel<128, false><<<a.B * a.Hq, 128, 0, s>>>(a);
    else decode_combine_kernel<64, false><<<a.B * a.Hq, 64, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_kpack_bf16(const KPackArgs &a, int d, hipStream_t s) {
    const long long total = (long long)a.n * (a.v ? d / 8 + d / 8 : d / 8);
    const unsigned gx = (unsigned)std::min<long long>((total + 255) / 256, 65535);
    dim3 grid(gx, (unsigned)(a.B * a.Hkv));
    if (d == 256) kpack_bf16_kernel<256><<<grid, 256, 0, s>>>(a);
    else if (d == 128) kpack_bf16_kernel<128><<<grid, 256, 0, s>>>(a);
    else kpack_bf16_kernel<64><<<grid, 256, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_paged_write_bf16(const PagedWriteArgs &a, int d, hipStream_t s) {
    const long long total = (long long)a.n * (d / 8 + d / 8);
    const unsigned gx = (unsigned)std::min<long long>((total + 255) / 256, 65535);
    dim3 grid(gx, (unsigned)(a.B * a.Hkv));
    if (d == 256) paged_write_bf16_kernel<256><<<grid, 256, 0, s>>>(a);
    else if (d == 128) paged_write_bf16_kernel<128><<<grid, 256, 0, s>>>(a);
    else paged_write_bf16_kernel<64><<<grid, 256, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_decode_paged_bf16(const DecodeArgs &a, int d, hipStream_t s) {
    launch_decode_qrot<true>(a, d, s);
    dim3 grid((unsigned)a.nsplit, (unsigned)(a.B * a.Hkv * a.n_slabs));
    // paged: x walks the batch's splits (at most budget + B of them), y = (kv head, slab)
    grid = dim3((unsigned)(a.split_budget + a.B), (unsigned)(a.Hkv * a.n_slabs));
    if (d == 256) decode_kcache_bf16_kernel<256, true><<<grid, 256, 0, s>>>(a);
    else if (d == 128) decode_kcache_bf16_kernel<128, true><<<grid, 256, 0, s>>>(a);
    else decode_kcache_bf16_kernel<64, true><<<grid, 256, 0, s>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (d == 256) decode_combine_kernel<256, true><<<a.B * a.Hq, 256, 0, s>>>(a);
    else if (d == 128) decode_combine_kernel<128, true><<<a.B * a.Hq, 128, 0, s>>>(a);
    else decode_combine_kernel<64, true><<<a.B * a.Hq, 64, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_decode_kcache_bf16(const DecodeArgs &a, int d, hipStream_t s) {
    launch_decode_qrot<false>(a, d, s);
    dim3 grid((unsigned)a.nsplit, (unsigned)(a.B * a.Hkv * a.n_slabs));
    if (d == 256) decode_kcache_bf16_kernel<256, false><<<grid, 256, 0, s>>>(a);
    else if (d == 128) decode_kcache_bf16_kernel<128, false><<<grid, 256, 0, s>>>(a);
    else decode_kcache_bf16_kernel<64, false><<<grid, 256, 0, s>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (d == 256) decode_combine_kernel<256, false><<<a.B * a.Hq, 256, 0, s>>>(a);
    else if (d == 128) decode_combine_kernel<128, false><<<a.B * a.Hq, 128, 0, s>>>(a);
    else decode_combine_kernel<64, false><<<a.B * a.Hq, 64, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_fill_zero_u64(unsigned long long *p, hipStream_t s) {
    fill_zero_u64_kernel<<<1, 1, 0, s>>>(p);
    return hipGetLastError();
}

hipError_t launch_prefill_qrot(const AttnArgs &a, int d, hipStream_t s) {
    const unsigned rows = (unsigned)((long long)a.B * a.Hq * a.Sq);
    if (d == 256) prefill_qrot_kernel<256><<<rows, 128, 0, s>>>(a);
    else if (d == 128) prefill_qrot_kernel<128><<<rows, 64, 0, s>>>(a);
    else prefill_qrot_kernel<64><<<rows, 32, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace atf

// Scratch of the entry point that allocates nothing (paged decode: counter,
// rotated queries, split partials).  Every GPU the library runs on holds its
// own copy for the life of the process; host code reaches it only through the
// address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[atf::kNoAllocScratchBytes];

namespace atf {

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];
}  // namespace

hipError_t noalloc_scratch(hipStream_t s, void **ptr) {
    *ptr = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    if (s != nullptr) {
        int sdev = -1;
        e = hipStreamGetDevice(s, &sdev);
        if (e != hipSuccess) return e;
        if (sdev != dev) return hipSuccess;  // *ptr stays NULL: the caller reports the mismatch
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace atf
