// Weight-streaming matrix-vector core for small batches (gfx950, wave64).
//
// Every weight byte is read from HBM once per step (Primer 1.2: decode time is
// the time to read the weights once; Unsloth article 二.3: int4 codes are
// expanded only in registers).  Rows are processed in pairs (two rows that one
// epilogue needs together: the two halves of a RoPE pair, a gate row and its
// up row, or two adjacent rows).  A pair's K axis is cut into units of
// 16 lanes x one 16-byte load per row, so each 16-lane DPP row streams 256
// contiguous bytes of each of its two rows per load.
//
// Work split.  The pairs of a pass are split evenly over workgroups; inside a
// workgroup the (pair, unit) grid is cut into one contiguous range per wave and
// then one contiguous range per 16-lane slot.  A slot accumulates in registers
// while its pair stays the same and parks the per-lane sum of a finished pair
// ("run") in a small register array; at the end of the pass the runs are
// summed over their 16 lanes with DPP rotations and written to LDS, and the
// per-pair totals are formed in slot order -- a fixed order, so results are
// bit-reproducible.
//
// Loads are software-pipelined: each lane keeps D units in flight in a ring of
// registers, and the ring runs ahead across pass boundaries of a phase.
//
// int4 unpack: a dword holds 8 codes c0..c7 (c0 lowest nibble).  OR-ing
// 0x6400 (fp16 1024.0) into the masked halves gives fp16 (1024 + c) for the
// nibbles at bits 0-3 / 16-19 and (1024 + 16 c) for bits 4-7 / 20-23 (likewise
// after one 8-bit shift), all exact.  The activations are staged in LDS as fp16
// pairs in the matching order, the odd ones pre-divided by 16 (exact), and
// v_dot2_f32_f16 accumulates in fp32.  The bias terms and the zero-point of 8
// come out as one per-32-input correction computed at staging time:
//   sum (c - 8) x = acc - (1032 * sum x_even + 1152 * sum a_odd)
// (a_odd = the stored x_odd / 16).  The bf16 group scale multiplies the unit's
// partial sum once.  This costs about 1.2 VALU operations per weight.
// fp16 range: each staged chunk is multiplied by a power of two 2^-e (e = 0
// unless its largest staged magnitude reaches 2^15), so every staged value is
// a finite fp16 whatever the activations' range; 2^e is stored beside the
// chunk's correction and multiplies the group scale (both exact).
#pragma once
#include "common.h"

enum { FMT_INT4_FAST = 0, FMT_INT4_GEN = 1, FMT_BF16_FAST = 2, FMT_BF16_GEN = 3 };
enum { KIND_ADJ = 0, KIND_TWO = 1, KIND_QKV = 2 };

struct DevMat {
    const uint8_t* data;       // int4 codes [n][k/2] or bf16 [n][k]
    const uint16_t* scales;    // bf16 [n][ngroups] (int4 only)
    int n, k, group, ngroups;
};

// One matrix-vector phase.
struct GemvTask {
    int kind;                  // KIND_*
    DevMat a, b, c;            // ADJ: a.  TWO: rows of a paired with rows of b.  QKV: q, k, v.
    int k;                     // inputs per row (all matrices of the task)
    int pitch_k;               // inputs per row in memory (k, or more when the task covers a K-chunk)
    int log2_group;            // fast int4 path: group = 1 << log2_group
    int head_dim;              // QKV pairing
    int total_pairs;
    int pass_pairs;            // pairs per pass (all workgroups together)
    int npasses;
    int young;                 // share of the younger wave of each SIMD in an 8-wave workgroup, percent
};

template <int FMT> struct FmtT;
template <> struct FmtT<FMT_INT4_FAST> { static constexpr int LANE_B = 16, LANE_W = 32, UNIT_W = 512; static constexpr bool INT4 = true; };
template <> struct FmtT<FMT_INT4_GEN>  { static constexpr int LANE_B = 4,  LANE_W = 8,  UNIT_W = 128; static constexpr bool INT4 = true; };
template <> struct FmtT<FMT_BF16_FAST> { static constexpr int LANE_B = 16, LANE_W = 8,  UNIT_W = 128; static constexpr bool INT4 = false; };
template <> struct FmtT<FMT_BF16_GEN>  { static constexpr int LANE_B = 4,  LANE_W = 2,  UNIT_W = 32;  static constexpr bool INT4 = false; };

// ---------------------------------------------------------------- LDS footprint of a staged activation
// int4: PREC planes of fp16 pairs [NB][K/2] (4 B each; plane 0 the fp16 value,
// plane 1 the fp16 of the remainder) + per chunk {correction, 2^e} [NB][K/LANE_W] fp32 pairs.
// bf16: fp32 [NB][K].
template <int FMT, int NB, int PREC>
__host__ __device__ constexpr int act_lds_bytes(int K) {
    return FmtT<FMT>::INT4 ? NB * (PREC * K * 2 + (K / FmtT<FMT>::LANE_W) * 8) : NB * K * 4;
}

// ---------------------------------------------------------------- pair -> rows
struct RowPtrs { const uint8_t* pa; const uint8_t* pb; const uint16_t* sa; const uint16_t* sb; };

// KND: the task's kind when the kernel knows it at compile time (then only
// that mapping is compiled), or -1 to read it from the task.
template <int FMT, int KND = -1>
I4D_DEVINL RowPtrs resolve_pair(const GemvTask& t, int pair) {
    // select by value (no pointer to a member of the kernel argument, which
    // would push the task into scratch memory)
    const int kind = KND >= 0 ? KND : t.kind;
    const uint8_t* da = t.a.data; const uint16_t* sa = t.a.scales; int ga = t.a.ngroups;
    const uint8_t* db; const uint16_t* sb; int gb;
    int ra, rb;
    if (kind == KIND_ADJ) {
        ra = 2 * pair;
        rb = min(2 * pair + 1, t.a.n - 1);
        db = da; sb = sa; gb = ga;
    } else if (kind == KIND_TWO) {
        ra = pair; rb = pair;
        db = t.b.data; sb = t.b.scales; gb = t.b.ngroups;
    } else {
        const int half = t.head_dim >> 1;
        const int npq = t.a.n >> 1, npk = t.b.n >> 1;
        int lp = pair;
        if (lp >= npq) {
            lp -= npq;
            if (lp >= npk) { lp -= npk; da = t.c.data; sa = t.c.scales; ga = t.c.ngroups; }
            else { da = t.b.data; sa = t.b.scales; ga = t.b.ngroups; }
        }
        const int head = lp >> __builtin_ctz(half), i = lp & (half - 1);     // head_dim is 64 or 128
        ra = head * t.head_dim + i;
        rb = ra + half;
        db = da; sb = sa; gb = ga;
    }
    const size_t row_bytes = FmtT<FMT>::INT4 ? (size_t)(t.pitch_k >> 1) : (size_t)t.pitch_k * 2;
    RowPtrs r;
    r.pa = da + (size_t)ra * row_bytes;
    r.pb = db + (size_t)rb * row_bytes;
    r.sa = FmtT<FMT>::INT4 ? sa + (size_t)ra * ga : nullptr;
    r.sb = FmtT<FMT>::INT4 ? sb + (size_t)rb * gb : nullptr;
    return r;
}

// ---------------------------------------------------------------- one buffered unit
// The registers of one unit are only written by loads: nothing is computed
// from them until the unit is consumed, so a load never forces a wait on
// itself and D units stay in flight.
template <int FMT> struct Unit;
template <> struct Unit<FMT_INT4_FAST> { u32x4 a, b; u32 sa, sb; };
template <> struct Unit<FMT_INT4_GEN>  { u32 a, b; u32 sa, sb; };
template <> struct Unit<FMT_BF16_FAST> { u32x4 a, b; };
template <> struct Unit<FMT_BF16_GEN>  { u32 a, b; };

template <class T> I4D_DEVINL T nt_load(const T* p) { return ld_g_nt(p); }

// Issue the loads of one unit.  `valid` = the unit exists; otherwise the
// loads read a fixed in-bounds address (the first bytes of the task's first
// matrix, cached after the first touch) and the unit is never consumed.  The
// loads are unconditional so the compiler can count them exactly.
template <int FMT>
I4D_DEVINL void load_unit(Unit<FMT>& u, const RowPtrs& rp, int seg, int lane16, int K, int log2g, int group,
                          bool valid, const uint8_t* dummy, const uint16_t* dummy_s) {
    typedef FmtT<FMT> F;
    int k0 = seg * F::UNIT_W + lane16 * F::LANE_W;          // first input of this lane's load
    if constexpr (FMT == FMT_INT4_GEN || FMT == FMT_BF16_GEN) valid = valid && (k0 < K);
    if constexpr (F::INT4) {
        const size_t off = (size_t)(k0 >> 1);
        const int gi = (FMT == FMT_INT4_FAST) ? (k0 >> log2g) : (k0 / group);
        const uint8_t* pa = valid ? rp.pa + off : dummy;
        const uint8_t* pb = valid ? rp.pb + off : dummy;
        const uint16_t* qa = valid ? rp.sa + gi : dummy_s;
        const uint16_t* qb = valid ? rp.sb + gi : dummy_s;
        if constexpr (FMT == FMT_INT4_FAST) {
            u.a = nt_load((const u32x4*)pa);
            u.b = nt_load((const u32x4*)pb);
            // The aligned 32-bit word that holds the bf16 scale (on this path
            // scale rows have an even length and a 4-byte aligned base): the
            // value of a 16-bit load is re-masked where the loop closes, and
            // that makes the compiler wait there for every load in flight.
            u.sa = ld_g((const u32*)((uintptr_t)qa & ~(uintptr_t)3));
            u.sb = ld_g((const u32*)((uintptr_t)qb & ~(uintptr_t)3));
        } else {
            u.a = nt_load((const u32*)pa);
            u.b = nt_load((const u32*)pb);
            u.sa = ld_g(qa);
            u.sb = ld_g(qb);
        }
    } else {
        const size_t off = (size_t)k0 * 2;
        const uint8_t* pa = valid ? rp.pa + off : dummy;
        const uint8_t* pb = valid ? rp.pb + off : dummy;
        if constexpr (FMT == FMT_BF16_FAST) {
            u.a = nt_load((const u32x4*)pa);
            u.b = nt_load((const u32x4*)pb);
        } else {
            u.a = nt_load((const u32*)pa);
            u.b = nt_load((const u32*)pb);
        }
    }
}

// ---------------------------------------------------------------- dot products of one unit
I4D_DEVINL h2 as_h2(u32 v) { return __builtin_bit_cast(h2, v); }

// (a & m) | o in one VALU operation.  gfx9 VOP3 encodings take no literal
// constants, so the compiler splits the expression into an AND and an OR; the
// mask comes in through a scalar register and the OR value through a vector
// register instead (one scalar operand per instruction is allowed).
I4D_DEVINL u32 and_or(u32 a, u32 m, u32 o) {
    u32 r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(m), "v"(o));
    return r;
}

// acc + sum over one dword of 8 codes, with act[4] the staged fp16 pairs.
I4D_DEVINL float dot8_int4(u32 w, const h2* act, float acc) {
    const u32 w8 = w >> 8;
    const u32 magic = 0x64006400u;
    acc = __builtin_amdgcn_fdot2(as_h2(and_or(w, 0x000F000Fu, magic)), act[0], acc, false);
    acc = __builtin_amdgcn_fdot2(as_h2(and_or(w, 0x00F000F0u, magic)), act[1], acc, false);
    acc = __builtin_amdgcn_fdot2(as_h2(and_or(w8, 0x000F000Fu, magic)), act[2], acc, false);
    acc = __builtin_amdgcn_fdot2(as_h2(and_or(w8, 0x00F000F0u, magic)), act[3], acc, false);
    return acc;
}

template <int FMT, int NB, int PREC>
I4D_DEVINL void consume_unit(const Unit<FMT>& u, const char* act_lds, int K, int log2g, int seg, int lane16,
                             float (&ra)[NB], float (&rb)[NB]) {
    typedef FmtT<FMT> F;
    if constexpr (F::INT4) {
        const int nchunk = K / F::LANE_W;
        int c = seg * 16 + lane16;                      // lane chunk index along K
        if (FMT == FMT_INT4_GEN) c = min(c, nchunk - 1);  // masked lanes read a valid chunk, scale 0
        const float2* corr = (const float2*)(act_lds + NB * PREC * K * 2);
        float sa, sb;
        if constexpr (FMT == FMT_INT4_FAST) {
            // the half of the scale word: the parity of the group index
            const bool odd = ((c * F::LANE_W) >> log2g) & 1;
            sa = __uint_as_float(odd ? (u.sa & 0xFFFF0000u) : (u.sa << 16));
            sb = __uint_as_float(odd ? (u.sb & 0xFFFF0000u) : (u.sb << 16));
        } else {
            // generic path: lanes past the end of K contribute nothing
            const bool live = seg * F::UNIT_W + lane16 * F::LANE_W < K;
            sa = live ? bf16_to_f32((uint16_t)u.sa) : 0.f;
            sb = live ? bf16_to_f32((uint16_t)u.sb) : 0.f;
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const float2 cr = corr[b * nchunk + c];         // {correction, 2^e of the chunk}
            float acca = -cr.x, accb = -cr.x;
#pragma unroll
            for (int pl = 0; pl < PREC; ++pl) {
                const h2* act = (const h2*)act_lds + (size_t)(pl * NB + b) * (K >> 1);
                if constexpr (FMT == FMT_INT4_FAST) {
                    const u32x4* ap = (const u32x4*)(act + c * 16);
                    u32x4 x0 = ap[0], x1 = ap[1], x2 = ap[2], x3 = ap[3];
                    h2 xa[16] = {as_h2(x0.x), as_h2(x0.y), as_h2(x0.z), as_h2(x0.w), as_h2(x1.x), as_h2(x1.y), as_h2(x1.z), as_h2(x1.w),
                                 as_h2(x2.x), as_h2(x2.y), as_h2(x2.z), as_h2(x2.w), as_h2(x3.x), as_h2(x3.y), as_h2(x3.z), as_h2(x3.w)};
                    acca = dot8_int4(u.a.x, xa + 0, acca);  accb = dot8_int4(u.b.x, xa + 0, accb);
                    acca = dot8_int4(u.a.y, xa + 4, acca);  accb = dot8_int4(u.b.y, xa + 4, accb);
                    acca = dot8_int4(u.a.z, xa + 8, acca);  accb = dot8_int4(u.b.z, xa + 8, accb);
                    acca = dot8_int4(u.a.w, xa + 12, acca); accb = dot8_int4(u.b.w, xa + 12, accb);
                } else {
                    const u32x4 x0 = *(const u32x4*)(act + c * 4);
                    h2 xa[4] = {as_h2(x0.x), as_h2(x0.y), as_h2(x0.z), as_h2(x0.w)};
                    acca = dot8_int4(u.a, xa, acca);
                    accb = dot8_int4(u.b, xa, accb);
                }
            }
            ra[b] = fmaf(sa * cr.y, acca, ra[b]);
            rb[b] = fmaf(sb * cr.y, accb, rb[b]);
        }
    } else {
        const float* act = (const float*)act_lds;
        int k0 = seg * F::UNIT_W + lane16 * F::LANE_W;
        const bool live = (FMT == FMT_BF16_FAST) || (k0 < K);
        if (FMT == FMT_BF16_GEN) k0 = min(k0, K - 2);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const float* xp = act + (size_t)b * K + k0;
            float acca = 0.f, accb = 0.f;
            if constexpr (FMT == FMT_BF16_FAST) {
                const f4 x0 = *(const f4*)xp, x1 = *(const f4*)(xp + 4);
                const float xv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
                const u32 wa[4] = {u.a.x, u.a.y, u.a.z, u.a.w};
                const u32 wb[4] = {u.b.x, u.b.y, u.b.z, u.b.w};
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    acca = fmaf(__uint_as_float(wa[d] << 16), xv[2 * d], acca);
                    acca = fmaf(__uint_as_float(wa[d] & 0xFFFF0000u), xv[2 * d + 1], acca);
                    accb = fmaf(__uint_as_float(wb[d] << 16), xv[2 * d], accb);
                    accb = fmaf(__uint_as_float(wb[d] & 0xFFFF0000u), xv[2 * d + 1], accb);
                }
            } else {
                acca = fmaf(__uint_as_float(u.a << 16), xp[0], __uint_as_float(u.a & 0xFFFF0000u) * xp[1]);
                accb = fmaf(__uint_as_float(u.b << 16), xp[0], __uint_as_float(u.b & 0xFFFF0000u) * xp[1]);
            }
            ra[b] += live ? acca : 0.f;
            rb[b] += live ? accb : 0.f;
        }
    }
}

// ---------------------------------------------------------------- activation staging
// Stage nb rows of `src` (fp32, row stride src_stride, K inputs) into LDS for
// NB batch slots (missing rows are zeros), optionally RMS-normalised with a bf16
// gain: h = x / sqrt(mean(x^2) + eps) * gain.
//
// Staging is split in two so that its global loads are issued before the
// weight loads (the vector-memory counter is in order: a wait for a load also
// waits for every load issued before it).  stage_issue() loads the first
// PRE_CHUNKS chunks of each thread into registers; stage_finish() does the
// rest.  `red` is NT/64*NB floats of LDS.
constexpr int PRE_CHUNKS = 1;

// PC: chunks per thread loaded up front (the rest are loaded, and waited
// for, while staging).
template <int FMT, int PC = PRE_CHUNKS>
struct StagePre {
    static constexpr int NV = FmtT<FMT>::INT4 ? FmtT<FMT>::LANE_W / 4 : 2;   // float4 loads per chunk
    static constexpr int CH = PC;
    f4 x[PC][NV];
    u32x4 g[PC][FmtT<FMT>::INT4 ? NV / 2 : 1];
};

// chunk geometry: int4 chunks are LANE_W inputs; bf16 chunks are 8 inputs
template <int FMT> I4D_DEVINL int stage_chunk_w() { return FmtT<FMT>::INT4 ? FmtT<FMT>::LANE_W : 8; }

template <int FMT, int NB, int NT>
I4D_DEVINL void stage_load_chunk(f4 (&xv)[StagePre<FMT>::NV], u32x4 (&gv)[FmtT<FMT>::INT4 ? StagePre<FMT>::NV / 2 : 1],
                                 const float* src, int src_stride, int K, int nb, const uint16_t* gain, int idx) {
    constexpr int NV = StagePre<FMT>::NV;
    const int cw = stage_chunk_w<FMT>();
    const int nchunk = K / cw;
    const int b = idx / nchunk, c = idx - b * nchunk;
    const int k0 = c * cw;
    // written by an earlier phase: either an earlier kernel, or -- in the
    // persistent kernel -- a buffer of this layer that no workgroup read
    // before it was written (so no L2 holds a stale copy of it)
    const f4* xp = (const f4*)(src + (size_t)min(b, nb - 1) * src_stride + k0);
#pragma unroll
    for (int i = 0; i < NV; ++i) xv[i] = ld_g(xp + i);
    if (gain != nullptr) {
        constexpr int NG = FmtT<FMT>::INT4 ? NV / 2 : 1;
#pragma unroll
        for (int i = 0; i < NG; ++i) gv[i] = ld_g((const u32x4*)(gain + k0) + i);
    }
}

template <int FMT, int NB, int NT, int PC = PRE_CHUNKS>
I4D_DEVINL void stage_issue(StagePre<FMT, PC>& pre, const float* src, int src_stride, int K, int nb, const uint16_t* gain) {
    const int nidx = NB * (K / stage_chunk_w<FMT>());
#pragma unroll
    for (int pc = 0; pc < PC; ++pc) {
        const int idx = min(i4d_tid() + pc * NT, nidx - 1);     // clamped: loads are unconditional
        stage_load_chunk<FMT, NB, NT>(pre.x[pc], pre.g[pc], src, src_stride, K, nb, gain, idx);
    }
}

// Write one chunk (already in registers) to LDS.
template <int FMT, int NB, int PREC>
I4D_DEVINL void stage_write_chunk(char* act_lds, const f4 (&xv)[StagePre<FMT>::NV],
                                  const u32x4 (&gv)[FmtT<FMT>::INT4 ? StagePre<FMT>::NV / 2 : 1],
                                  int K, int nb, bool has_gain, const float (&rs)[NB], int idx) {
    typedef FmtT<FMT> F;
    const int cw = stage_chunk_w<FMT>();
    const int nchunk = K / cw;
    const int b = idx / nchunk, c = idx - b * nchunk;
    const int k0 = c * cw;
    float scale = 0.f;
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) if (bb == b && b < nb) scale = rs[bb];
    if constexpr (F::INT4) {
        h2* act = (h2*)act_lds;
        float2* corr = (float2*)(act_lds + NB * PREC * K * 2);
        // staged values a (odd positions pre-divided by 16, exact), then the
        // chunk's power of two: largest |a| below 2^15 after it
        float av[F::LANE_W];
        float amax = 0.f;
#pragma unroll
        for (int q = 0; q < F::LANE_W; ++q) {
            float v = xv[q >> 2][q & 3] * scale;
            if (has_gain) {
                const u32 gw = gv[q >> 3][(q >> 1) & 3];
                v *= __uint_as_float((q & 1) ? (gw & 0xFFFF0000u) : (gw << 16));
            }
            av[q] = (q & 1) ? v * 0.0625f : v;
            amax = fmaxf(amax, fabsf(av[q]));
        }
        int ex = 0;
        (void)frexpf(amax, &ex);                      // amax < 2^ex (0 for amax = 0; inf/NaN stay as they are)
        const int sh = max(ex - 15, 0);
        const float down = ldexpf(1.f, -sh);
        double ce = 0.0;
#pragma unroll
        for (int d = 0; d < F::LANE_W / 8; ++d) {
            // hi = fp16(a), lo = fp16(a - hi) when two planes are used
            _Float16 hi[8], lo[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float a = av[d * 8 + e] * down;
                hi[e] = (_Float16)a;
                lo[e] = (_Float16)(a - (float)hi[e]);
                const double w = (e & 1) ? 1152.0 : 1032.0;
                ce += w * ((double)hi[e] + (PREC > 1 ? (double)lo[e] : 0.0));
            }
            h2* dst = act + (size_t)b * (K >> 1) + (size_t)((k0 >> 1) + 4 * d);
            dst[0] = h2{hi[0], hi[4]};
            dst[1] = h2{hi[1], hi[5]};
            dst[2] = h2{hi[2], hi[6]};
            dst[3] = h2{hi[3], hi[7]};
            if (PREC > 1) {
                h2* dl = dst + (size_t)NB * (K >> 1);
                dl[0] = h2{lo[0], lo[4]};
                dl[1] = h2{lo[1], lo[5]};
                dl[2] = h2{lo[2], lo[6]};
                dl[3] = h2{lo[3], lo[7]};
            }
        }
        corr[b * nchunk + c] = float2{(float)ce, ldexpf(1.f, sh)};
    } else {
        float* act = (float*)act_lds + (size_t)b * K + k0;
        const u32x4 gw = gv[0];
        const u32 gws[4] = {gw.x, gw.y, gw.z, gw.w};
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            float v = xv[q >> 2][q & 3] * scale;
            if (has_gain) v *= __uint_as_float((q & 1) ? (gws[q >> 1] & 0xFFFF0000u) : (gws[q >> 1] << 16));
            act[q] = v;
        }
    }
}

template <int FMT, int NB, int NT, int PREC, int PC = PRE_CHUNKS>
I4D_DEVINL void stage_finish(const StagePre<FMT, PC>& pre, char* act_lds, const float* src, int src_stride, int K, int nb,
                             const uint16_t* gain, float eps, float* red) {
    const int tid = i4d_tid();
    const int nidx = NB * (K / stage_chunk_w<FMT>());
    float rs[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) rs[b] = 1.0f;
    if (gain != nullptr) {
        // sum of squares per batch row: prefetched chunks from registers, the rest from memory
        float ss[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) ss[b] = 0.f;
        const int nchunk = K / stage_chunk_w<FMT>();
#pragma unroll
        for (int pc = 0; pc < PC; ++pc) {
            const int idx = tid + pc * NT;
            if (idx < nidx) {
                f4 acc = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int i = 0; i < StagePre<FMT>::NV; ++i) acc += pre.x[pc][i] * pre.x[pc][i];
                const float v = (acc.x + acc.y) + (acc.z + acc.w);
#pragma unroll
                for (int b = 0; b < NB; ++b) if (b == idx / nchunk) ss[b] += v;
            }
        }
        for (int idx = tid + PC * NT; idx < nidx; idx += NT) {
            f4 xv[StagePre<FMT>::NV];
            u32x4 gv[FmtT<FMT>::INT4 ? StagePre<FMT>::NV / 2 : 1];
            stage_load_chunk<FMT, NB, NT>(xv, gv, src, src_stride, K, nb, nullptr, idx);
            f4 acc = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < StagePre<FMT>::NV; ++i) acc += xv[i] * xv[i];
            const float v = (acc.x + acc.y) + (acc.z + acc.w);
#pragma unroll
            for (int b = 0; b < NB; ++b) if (b == idx / nchunk) ss[b] += v;
        }
#pragma unroll
        for (int b = 0; b < NB; ++b)
            for (int m = 32; m >= 1; m >>= 1) ss[b] += shfl_xor_f(ss[b], m);
        const int wave = tid >> 6;
        if ((tid & 63) == 0) {
#pragma unroll
            for (int b = 0; b < NB; ++b) red[wave * NB + b] = ss[b];
        }
        __syncthreads();
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            float t = 0.f;
            for (int w = 0; w < NT / 64; ++w) t += red[w * NB + b];
            rs[b] = 1.0f / sqrtf(t / (float)K + eps);
        }
        __syncthreads();   // red may be reused by the caller
    }
#pragma unroll
    for (int pc = 0; pc < PC; ++pc) {
        const int idx = tid + pc * NT;
        if (idx < nidx) stage_write_chunk<FMT, NB, PREC>(act_lds, pre.x[pc], pre.g[pc], K, nb, gain != nullptr, rs, idx);
    }
    for (int idx = tid + PC * NT; idx < nidx; idx += NT) {
        f4 xv[StagePre<FMT>::NV];
        u32x4 gv[FmtT<FMT>::INT4 ? StagePre<FMT>::NV / 2 : 1];
        stage_load_chunk<FMT, NB, NT>(xv, gv, src, src_stride, K, nb, gain, idx);
        stage_write_chunk<FMT, NB, PREC>(act_lds, xv, gv, K, nb, gain != nullptr, rs, idx);
    }
}

// ---------------------------------------------------------------- schedule arithmetic
// Pairs of pass p owned by workgroup w (32-bit: pairs * workgroups < 2^31).
I4D_DEVINL void pass_pairs_of(const GemvTask& t, int pass, int w, int nwg, int& q0, int& q1) {
    const int pb = pass * t.pass_pairs;
    const int np = min(t.total_pairs, pb + t.pass_pairs) - pb;
    q0 = pb + (w * np) / nwg;
    q1 = pb + ((w + 1) * np) / nwg;
}

// First unit of wave w when U units are split over NW waves.  With two
// waves per SIMD (8-wave workgroups) the sequencer issues from the older wave
// first: given equal shares, waves 0-3 finish about 1.4x sooner than waves
// 4-7.  So each younger wave gets `young` percent of its SIMD's share (the
// task's young; 50 = an even split).
template <int NW>
__host__ __device__ inline int wave_cut(int U, int w, int young) {
    if constexpr (NW == 8) {
        const int c = w <= 4 ? w * (100 - young) : 4 * (100 - young) + (w - 4) * young;
        return (int)(((long long)U * c) / 400);
    } else {
        return (w * U) / NW;
    }
}

// Unit range of 16-lane slot s (wave s/4, slot s%4) among U units of a workgroup;
// n_it = iterations every slot of that wave runs (the longest slot's count).
template <int NW>
I4D_DEVINL void slot_range(int U, int s, int young, int& u0, int& u1, int& n_it) {
    const int w = s >> 2, t = s & 3;
    const int wu0 = wave_cut<NW>(U, w, young), wu1 = wave_cut<NW>(U, w + 1, young);
    const int n = wu1 - wu0;
    u0 = wu0 + (t * n) / 4;
    u1 = wu0 + ((t + 1) * n) / 4;
    n_it = (n + 3) / 4;
}

// Per-lane position of the loader inside one pass.
struct LoadCursor {
    int u, u1;         // next unit to load, end of the slot's range
    int pair, seg;     // of unit u
    RowPtrs rp;
};

template <int FMT, int KND = -1>
I4D_DEVINL void cursor_begin(LoadCursor& lc, const GemvTask& t, int q0, int u0, int u1, int S) {
    lc.u = u0; lc.u1 = u1;
    const int ql = u0 / S;
    lc.pair = q0 + ql;
    lc.seg = u0 - ql * S;
    lc.rp = resolve_pair<FMT, KND>(t, u0 < u1 ? lc.pair : 0);
}

// Load the slot's next unit into dst (if any) and advance.
template <int FMT, int KND = -1>
I4D_DEVINL void cursor_load(LoadCursor& lc, Unit<FMT>& dst, const GemvTask& t, int S, int lane16) {
    const bool valid = lc.u < lc.u1;
    load_unit<FMT>(dst, lc.rp, lc.seg, lane16, t.k, t.log2_group, t.a.group, valid, t.a.data, t.a.scales);
    if (valid) {
        ++lc.u;
        if (++lc.seg == S) {
            lc.seg = 0;
            ++lc.pair;
            if (lc.u < lc.u1) lc.rp = resolve_pair<FMT, KND>(t, lc.pair);
        }
    }
}

// ---------------------------------------------------------------- the pass loop
// The load ring of one workgroup lane plus the geometry of the pass it is
// loading.  A ring can be primed for a phase (gemv_prime) long before the
// phase runs -- e.g. before the grid barrier that precedes it -- because
// weights do not depend on the previous phase.
template <int FMT, int D>
struct GemvPipe {
    Unit<FMT> ring[D];
    LoadCursor lc;
    int q0, q1, u0, u1, n_it;     // pass-0 geometry of the primed phase
};

// Issue the first D units of pass 0 of task t into the ring.
template <int FMT, int NT, int D, int KND = -1>
I4D_DEVINL void gemv_prime(GemvPipe<FMT, D>& P, const GemvTask& t, int w, int nwg) {
    constexpr int NW = NT / 64;
    const int slot = i4d_tid() >> 4, lane16 = i4d_tid() & 15;
    const int S = (t.k + FmtT<FMT>::UNIT_W - 1) / FmtT<FMT>::UNIT_W;
    pass_pairs_of(t, 0, w, nwg, P.q0, P.q1);
    slot_range<NW>((P.q1 - P.q0) * S, slot, t.young, P.u0, P.u1, P.n_it);
    cursor_begin<FMT, KND>(P.lc, t, P.q0, P.u0, P.u1, S);
#pragma unroll
    for (int i = 0; i < D; ++i) cursor_load<FMT, KND>(P.lc, P.ring[i], t, S, lane16);
}

struct NoNext { I4D_DEVINL void operator()() {} };

// Run every pass of task `t` for workgroup w, the ring P already primed
// for t.  Activations must already be staged in act_lds.  For each pass:
//   epi(pass, pair, b, va, vb)   -- per (pair, batch slot) results, pair in [q0, q1)
//   epi.end_pass(pass, q0, q1)   -- after all epilogue calls of the pass
// After the last pass's loads are consumed, next() may prime the ring for the
// following phase; its loads are then in flight during this epilogue.
// LDS: act_lds (staged activations), part_lds (NS*MAXJ*NB*2 floats + 2*NS ints).
template <int FMT, int NB, int PREC, int NT, int D, int MAXJ, int KND = -1, class Epi, class Next>
I4D_DEVINL void gemv_passes(GemvPipe<FMT, D>& P, const GemvTask& t, int w, int nwg, const char* act_lds, float* part_lds,
                            Epi& epi, Next& next) {
    constexpr int NW = NT / 64, NS = NT / 16;
    typedef FmtT<FMT> F;
    const int tid = i4d_tid();
    const int slot = tid >> 4, lane16 = tid & 15;
    const int S = (t.k + F::UNIT_W - 1) / F::UNIT_W;
    int* slot_info = (int*)(part_lds + NS * MAXJ * NB * 2);     // [NS][2]: first local pair, runs

    for (int pass = 0; pass < t.npasses; ++pass) {
        const int n_itp = ((P.n_it + D - 1) / D) * D;
        float ra[NB], rb[NB], da[MAXJ][NB], db[MAXJ][NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) { ra[b] = 0.f; rb[b] = 0.f; }
#pragma unroll
        for (int j = 0; j < MAXJ; ++j)
#pragma unroll
            for (int b = 0; b < NB; ++b) { da[j][b] = 0.f; db[j][b] = 0.f; }
        int run = 0;
        const int first_local = P.u0 / S;
        int seg = P.u0 - first_local * S;
        int u = P.u0;
        const int u1 = P.u1;

        for (int itb = 0; itb < n_itp; itb += D) {
#pragma unroll
            for (int i = 0; i < D; ++i) {
                if (u < u1) {
                    consume_unit<FMT, NB, PREC>(P.ring[i], act_lds, t.k, t.log2_group, seg, lane16, ra, rb);
                    ++u;
                    if (++seg == S) {   // this pair's run is complete: park it
                        seg = 0;
#pragma unroll
                        for (int j = 0; j < MAXJ; ++j)
                            if (j == run)
#pragma unroll
                                for (int b = 0; b < NB; ++b) { da[j][b] = ra[b]; db[j][b] = rb[b]; }
#pragma unroll
                        for (int b = 0; b < NB; ++b) { ra[b] = 0.f; rb[b] = 0.f; }
                        ++run;
                    }
                }
                cursor_load<FMT, KND>(P.lc, P.ring[i], t, S, lane16);
                // keep each unit's LDS reads next to their use: hoisting the
                // activation reads of later units costs registers, not time
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if (seg != 0) {      // a partially covered last pair
#pragma unroll
            for (int j = 0; j < MAXJ; ++j)
                if (j == run)
#pragma unroll
                    for (int b = 0; b < NB; ++b) { da[j][b] = ra[b]; db[j][b] = rb[b]; }
            ++run;
        }
        const int this_q0 = P.q0, this_q1 = P.q1;
        // next pass (or next phase): its first D units fly during this epilogue
        if (pass + 1 < t.npasses) {
            pass_pairs_of(t, pass + 1, w, nwg, P.q0, P.q1);
            slot_range<NW>((P.q1 - P.q0) * S, slot, t.young, P.u0, P.u1, P.n_it);
            cursor_begin<FMT, KND>(P.lc, t, P.q0, P.u0, P.u1, S);
#pragma unroll
            for (int i = 0; i < D; ++i) cursor_load<FMT, KND>(P.lc, P.ring[i], t, S, lane16);
        } else {
            next();
        }
        // 16-lane sums of every run, written by lane 0 of the slot
#pragma unroll
        for (int j = 0; j < MAXJ; ++j)
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const float sa = row16_sum(da[j][b]);
                const float sb = row16_sum(db[j][b]);
                if (lane16 == 0 && j < run) {
                    float* p = part_lds + ((slot * MAXJ + j) * NB + b) * 2;
                    p[0] = sa; p[1] = sb;
                }
            }
        if (lane16 == 0) { slot_info[2 * slot] = first_local; slot_info[2 * slot + 1] = min(run, MAXJ); }
        __syncthreads();
        // per-pair totals: one 16-lane DPP row per (pair, batch slot), lane i
        // reading the slots i, i+16, ..; a fixed rotation tree sums them
        const int npairs = this_q1 - this_q0;
        const int grp = tid >> 4;
        for (int base = 0; base < npairs * NB; base += NT / 16) {
            const int idx = base + grp;
            const int ql = idx / NB, b = idx - ql * NB;
            float va = 0.f, vb = 0.f;
            if (idx < npairs * NB) {
                for (int s2 = lane16; s2 < NS; s2 += 16) {
                    const int j = ql - slot_info[2 * s2];
                    if (j >= 0 && j < slot_info[2 * s2 + 1]) {
                        const float* p = part_lds + ((s2 * MAXJ + j) * NB + b) * 2;
                        va += p[0]; vb += p[1];
                    }
                }
            }
            va = row16_sum(va);
            vb = row16_sum(vb);
            if (lane16 == 0 && idx < npairs * NB) epi(pass, this_q0 + ql, b, va, vb);
        }
        epi.end_pass(pass, this_q0, this_q1);
        __syncthreads();
    }
}

// One whole phase in a single kernel: activation loads are issued first, then
// the weight ring, then the activations are staged (waiting only for their own
// loads), then every pass runs.
template <int FMT, int NB, int PREC, int NT, int D, int MAXJ, int KND, class Stage, class Epi>
I4D_DEVINL void gemv_run(const GemvTask& t, int w, int nwg, char* act_lds, float* part_lds, Stage& stage, Epi& epi) {
    typename Stage::Pre pre;
    stage.issue(pre);
    GemvPipe<FMT, D> P;
    gemv_prime<FMT, NT, D, KND>(P, t, w, nwg);
    stage.finish(pre);
    __syncthreads();
    NoNext nn;
    gemv_passes<FMT, NB, PREC, NT, D, MAXJ, KND>(P, t, w, nwg, act_lds, part_lds, epi, nn);
}

// Largest number of runs any slot can see in a pass of `pairs_per_wg` pairs
// with S units per pair (host-side sizing of passes).
__host__ inline int gemv_max_runs(int pairs_per_wg, int S, int nw, int young) {
    const long long U = (long long)pairs_per_wg * S;
    long long wave_units = (U + nw - 1) / nw;
    if (nw == 8) wave_units = (U * (100 - std::min(young, 50)) + 399) / 400 + 1;
    const long long slot_units = (wave_units + 3) / 4;
    return (int)((slot_units + S - 1) / S) + 1;
}
