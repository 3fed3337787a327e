// Batch-1 decode expert FFN (bf16 path): one token, k touched experts plus the
// always-on shared expert.  The layer is a pure weight stream -- every weight
// byte is used once -- so the kernels are built around HBM bandwidth:
//
//  * a persistent grid sized to the resident capacity of the chip;
//  * every wave owns one contiguous range of matrix rows: no cross-wave
//    dependency, so waves never wait on each other in the row loop;
//  * rows are split between "routed" waves (Q2K or MXFP4 rows) and "shared"
//    waves (bf16 rows) so that every wave streams about the same number of
//    bytes (the host picks the split); the roles are interleaved over the wave
//    ids so every CU gets both the VALU-heavy 2-bit rows and the cheap bf16
//    rows;
//  * the token's activations are turned once into the operands the row loop
//    needs (Q2K: the pre-scaled bf16 pairs and per-group sums described in
//    ffn_gemv.hip; MXFP4 and bf16: plain bf16 pairs): in LDS, once per
//    workgroup, for the routed rows of the up pass (one activation row serves
//    every routed row); in registers otherwise;
//  * the loads of row i+1 are in flight while row i is reduced.
//
// Up pass: gate and up rows of the k experts and of the shared expert, each a
// full dot product with x, written as fp32 (shared rows in two K-halves so
// that a shared piece costs about as much as a few routed rows).  Down pass:
// h = silu(g) * u rounded to bf16 (summing the shared halves), then the down
// rows, written as the bf16 expert_out / shared_out of the API.
#include "formats.hpp"
#include "launch.hpp"

namespace ds4 {

constexpr uint32_t D1_BF16_128X2 = 0x43004300u;
constexpr int D1_KS_UP = 2;     // K-pieces of a shared up row

struct D1Args {
    int K, rows, nmat, k, E;            // routed matrices: nmat x k experts x rows x K
    size_t dstride, sstride;            // per-expert bytes (data, MXFP4 scales)
    const uint8_t* m[2];
    const uint8_t* sc[2];
    int Ks, rows_s, ks;                 // shared: nmat x rows_s rows of Ks, split in ks pieces
    const uint16_t* sm[2];
    const int32_t* active;              // slot -> expert (active[1 + slot])
    const uint16_t* x;                  // up: x[H] bf16
    const float* gu_r;                  // down: routed [k][2][F] fp32 (g, u)
    const float* gu_s;                  // down: shared [2][Fs][KS_UP] fp32 partials
    float* out_r;                       // up: routed [k][2][F]
    float* out_s;                       // up: shared [2][Fs][KS_UP]
    uint16_t* eo;                       // down: expert_out [k][H]
    uint16_t* so;                       // down: shared_out [H]
    int NW, NWs;                        // waves in the grid / of them in the shared role
};

__device__ __forceinline__ float d1_dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

template <int SEL>
__device__ __forceinline__ uint32_t d1_fp4x2(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, SEL));
}

// Q2K rows are streamed through a per-wave LDS ring: 1 KB chunks (64 lanes x
// 16 contiguous bytes) loaded straight into LDS by global_load_lds_dwordx4,
// D1_DEPTH chunks ahead of the row being decoded.  Wide contiguous loads keep
// the stream at the chip's bandwidth; the 84-byte blocks are then read from
// LDS in whatever lane layout the decode wants.
constexpr int D1_RING = 8;                  // chunks per wave ring (power of two)
constexpr int D1_DEPTH = 4;                 // chunks in flight ahead of the current row
constexpr int D1_RING_BYTES = D1_RING * 1024;

// 64 lanes x 16 B from global memory straight into LDS at lds_chunk + 16*lane.
// Issued through inline asm so that the compiler's wait-count pass does not
// treat every later LDS read as a possible alias of the transfer (it would
// wait for all outstanding loads); this code waits with explicit counts.
// The lgkmcnt(0) makes earlier LDS reads of the slot complete first.
__device__ __forceinline__ void d1_dma16(const uint8_t* g, uint8_t* lds_chunk) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds_chunk);
    asm volatile(
        "s_waitcnt lgkmcnt(0)\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, off"
        :
        : "v"(g), "s"(m0)
        : "memory", "m0");
}

// Wait until at most n of this wave's vector-memory operations are
// outstanding (n < D1_DEPTH); the memory clobber keeps LDS reads after it.
__device__ __forceinline__ void d1_wait_vm(int n) {
    switch (n) {
        case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
        case 1: asm volatile("s_waitcnt vmcnt(1)" ::: "memory"); break;
        case 2: asm volatile("s_waitcnt vmcnt(2)" ::: "memory"); break;
        default: asm volatile("s_waitcnt vmcnt(3)" ::: "memory"); break;
    }
}

// Role and row range of wave w: shared waves are spread evenly over the wave
// ids; each role splits its rows evenly over its waves.
__device__ __forceinline__ void d1_range(int w, int NW, int NWs, int Rs, int Rr, bool& shared, int& r0, int& r1) {
    const int before = (int)(((long long)w * NWs) / NW);
    const int upto = (int)(((long long)(w + 1) * NWs) / NW);
    shared = upto > before;
    if (shared) {
        r0 = (int)(((long long)before * Rs) / NWs);
        r1 = (int)(((long long)(before + 1) * Rs) / NWs);
    } else {
        const int NWr = NW - NWs;
        const int wr = w - before;
        r0 = (int)(((long long)wr * Rr) / NWr);
        r1 = (int)(((long long)(wr + 1) * Rr) / NWr);
    }
}

// Activation element c of the pass's input row, as the bf16 value it is.
template <bool UP>
__device__ __forceinline__ float d1_act(const D1Args& a, int slot, int c, bool shared) {
    if (UP) return bf16_to_f32(a.x[c]);
    float g, u;
    if (shared) {
        const int Fs = a.Ks;
        g = 0.0f;
        u = 0.0f;
#pragma unroll
        for (int p = 0; p < D1_KS_UP; ++p) {
            g += a.gu_s[((size_t)0 * Fs + c) * D1_KS_UP + p];
            u += a.gu_s[((size_t)1 * Fs + c) * D1_KS_UP + p];
        }
    } else {
        const int F = a.K;
        g = a.gu_r[((size_t)slot * 2 + 0) * F + c];
        u = a.gu_r[((size_t)slot * 2 + 1) * F + c];
    }
    return bf16_to_f32(f32_to_bf16(silu_f32(g) * u));      // h is rounded to bf16
}

// Q2K operands of one 16-element group: 8 pre-scaled bf16 pairs, C and S.
template <bool UP>
__device__ __forceinline__ void d1_q2k_operands(const D1Args& a, int slot, int G, uint32_t xq[8], float& C,
                                                float& S) {
    float xv[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) xv[c] = d1_act<UP>(a, slot, 16 * G + c, false);
    float ssum = 0.0f, csum = 0.0f;
#pragma unroll
    for (int c = 0; c < 16; ++c) ssum += xv[c];
#pragma unroll
    for (int pi = 0; pi < 8; ++pi) {
        const float s = (pi % 3 == 0) ? 1.0f : ((pi % 3 == 1) ? 0.25f : 0.0625f);
        const float a0 = xv[pi] * s, a1 = xv[pi + 8] * s;
        xq[pi] = pack_bf16x2(a0, a1);     // exact: power-of-two scaling of bf16 values
        csum += a0 + a1;
    }
    C = 128.0f * csum;
    S = ssum;
}

// One Q2K group: y + sum over its 16 weights of w * x, from the code dword,
// the scale byte, the d/dmin dword and the group's operands.
__device__ __forceinline__ float d1_q2k_group(uint32_t c, uint32_t sm, uint32_t dd, const uint32_t* xq, float C,
                                              float S, float y) {
    const uint32_t c6 = c >> 6, c12 = c >> 12;
    float acc = -C;
    acc = d1_dot2((c & 0x00030003u) | D1_BF16_128X2, xq[0], acc);
    acc = d1_dot2((c & 0x000C000Cu) | D1_BF16_128X2, xq[1], acc);
    acc = d1_dot2((c & 0x00300030u) | D1_BF16_128X2, xq[2], acc);
    acc = d1_dot2((c6 & 0x00030003u) | D1_BF16_128X2, xq[3], acc);
    acc = d1_dot2((c6 & 0x000C000Cu) | D1_BF16_128X2, xq[4], acc);
    acc = d1_dot2((c6 & 0x00300030u) | D1_BF16_128X2, xq[5], acc);
    acc = d1_dot2((c12 & 0x00030003u) | D1_BF16_128X2, xq[6], acc);
    acc = d1_dot2((c12 & 0x000C000Cu) | D1_BF16_128X2, xq[7], acc);
    const float d = half_bits_to_f32(dd & 0xFFFFu);
    const float dmin = half_bits_to_f32(dd >> 16);
    y = fmaf(d * (float)(sm & 15u), acc, y);
    return fmaf(-dmin * (float)(sm >> 4), S, y);
}

// One MXFP4 block: y + sum over its 32 weights of w * x.
__device__ __forceinline__ float d1_mx_block(const u32x4& cw, uint32_t sv, const uint32_t* xp, float y) {
    float acc = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        acc = d1_dot2(d1_fp4x2<0>(cw[q]), xp[4 * q + 0], acc);
        acc = d1_dot2(d1_fp4x2<1>(cw[q]), xp[4 * q + 1], acc);
        acc = d1_dot2(d1_fp4x2<2>(cw[q]), xp[4 * q + 2], acc);
        acc = d1_dot2(d1_fp4x2<3>(cw[q]), xp[4 * q + 3], acc);
    }
    return y + ldexpf(acc, (int)sv - 127);
}

// Routed row index -> (slot, matrix, row within the matrix).
__device__ __forceinline__ void d1_split(const D1Args& a, int idx, int& slot, int& mat, int& r) {
    const int per_slot = a.nmat * a.rows;
    slot = idx / per_slot;
    const int rem = idx - slot * per_slot;
    mat = rem / a.rows;
    r = rem - mat * a.rows;
}

// Row results of a wave, kept in registers (lane j of a 64-row window holds
// the window's row j) and written with one coalesced store per window.  A
// store per row would be counted by the next row's wait on loads (stores and
// loads share the vector-memory counter) and expose a store round trip on
// every row.
struct D1Results {
    float v = 0.0f;
    int base = 0;       // first row of the window (wave-relative)
    __device__ __forceinline__ void put(int jw, float y, int lane) {
        if (lane == (jw & 63)) v = y;
    }
    // Flush if row jw closes a window or is the wave's last row.
    template <typename Store>
    __device__ __forceinline__ void maybe_flush(int jw, int nrows, int lane, Store store) {
        if ((jw & 63) == 63 || jw == nrows - 1) {
            if (lane <= (jw & 63)) store(base + lane, v);
            base = jw + 1;
        }
    }
};

// Loads of one routed row for this lane's units (Q2K groups / MXFP4 blocks).
template <int FMT, int UPL>
struct D1Row {
    u32x4 cw[FMT == 1 ? 1 : UPL];
    uint32_t c[UPL], s[UPL], d[UPL];
    int slot;
};

template <int FMT, int UPL>
__device__ __forceinline__ void d1_load_row(const D1Args& a, int idx, int lane, D1Row<FMT, UPL>& b) {
    const int NU = FMT == 1 ? a.K / 16 : a.K / 32;
    int mat, r;
    d1_split(a, idx, b.slot, mat, r);
    const int e = a.active[1 + b.slot];
    const uint8_t* base = a.m[mat] + (size_t)e * a.dstride;
#pragma unroll
    for (int i = 0; i < UPL; ++i) {
        // unconditional loads (lanes past the row re-read its last unit and
        // are skipped in the arithmetic): exact wait counts for the compiler
        const int u = min(lane + WAVE * i, NU - 1);
        if (FMT == 1) {
            const uint8_t* blk = base + ((size_t)r * (NU / 16) + (u >> 4)) * Q2K_BLOCK_BYTES;
            b.c[i] = ld_u32(blk + 16 + 4 * (u & 15));
            b.s[i] = blk[u & 15];
            b.d[i] = ld_u32(blk + 80);
        } else {
            const size_t fb = (size_t)r * NU + u;
            b.cw[i] = *reinterpret_cast<const u32x4*>(base + fb * 16);
            b.s[i] = a.sc[mat][(size_t)e * a.sstride + fb];
        }
    }
}

// ---------------------------------------------------------------------------
// LDS image of the up pass's operands (one token, all of K):
//   Q2K:   xq[2][NG] u32x4 (pairs 0-3 / 4-7 of group G), cs[NG] float2 (C, S)
//   MXFP4: xp[4][NB] u32x4 (elements 8v .. 8v+7 of block B)
// followed by x itself (bf16 [K]) for the shared rows.
template <int FMT>
__host__ __device__ constexpr size_t d1_up_image_bytes(int K) {
    return FMT == 1 ? (size_t)(K / 16) * 40 : (size_t)K * 2;
}

template <int FMT>
__device__ void d1_stage_up_lds(const D1Args& a, uint8_t* lds) {
    {
        u32x4* xs = reinterpret_cast<u32x4*>(lds + d1_up_image_bytes<FMT>(a.K));
        for (int c = threadIdx.x; c < a.K / 8; c += blockDim.x) xs[c] = reinterpret_cast<const u32x4*>(a.x)[c];
    }
    if (FMT == 1) {
        const int NG = a.K / 16;
        u32x4* xq = reinterpret_cast<u32x4*>(lds);
        float2* cs = reinterpret_cast<float2*>(lds + (size_t)NG * 32);
        for (int G = threadIdx.x; G < NG; G += blockDim.x) {
            uint32_t q[8];
            float C, S;
            d1_q2k_operands<true>(a, 0, G, q, C, S);
            xq[G] = u32x4{q[0], q[1], q[2], q[3]};
            xq[NG + G] = u32x4{q[4], q[5], q[6], q[7]};
            cs[G] = float2{C, S};
        }
    } else {
        const int NB = a.K / 32;
        u32x4* xp = reinterpret_cast<u32x4*>(lds);
        for (int i = threadIdx.x; i < NB * 4; i += blockDim.x) {
            const int B = i >> 2, v = i & 3;
            xp[v * NB + B] = *reinterpret_cast<const u32x4*>(a.x + 32 * B + 8 * v);
        }
    }
}

// Routed Q2K rows, streamed through the wave's LDS ring.  Lane l decodes
// groups l, l+64, ... of each row; up pass operands from the workgroup's LDS
// image, down pass operands in registers (rebuilt per expert).
template <bool UP, int UPL>
__device__ void d1_routed_q2k(const D1Args& a, int r0, int r1, int lane, const uint8_t* img, uint8_t* ring) {
    const int NG = a.K / 16;
    const int RB = a.K / 256 * Q2K_BLOCK_BYTES;            // bytes per row
    constexpr int RU = UP ? 1 : UPL;
    uint32_t xq[RU][8];
    float Cg[RU], Sg[RU];
    int cur_slot = -1;
    D1Results res;
    auto store = [&](int jw, float y) {
        if (UP) a.out_r[r0 + jw] = y;
        else a.eo[r0 + jw] = (uint16_t)f32_to_bf16(y);
    };
    int idx = r0;
    while (idx < r1) {
        int slot, mat, r;
        d1_split(a, idx, slot, mat, r);
        const int nrows = min(r1 - idx, a.rows - r);        // rows of this matrix in the range
        const uint8_t* src = a.m[mat] + (size_t)a.active[1 + slot] * a.dstride + (size_t)r * RB;
        const int nbytes = nrows * RB;
        const int nchunks = (nbytes + 1023) >> 10;
        if (!UP && slot != cur_slot) {                      // uniform: a new expert's h
#pragma unroll
            for (int i = 0; i < RU; ++i) {
                const int G = lane + WAVE * i;
                if (G < NG) d1_q2k_operands<false>(a, slot, G, xq[i], Cg[i], Sg[i]);
            }
            cur_slot = slot;
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");    // nothing older may count below
        int issued = 0;
        auto issue_upto = [&](int last) {
            for (; issued <= last && issued < nchunks; ++issued) {
                const int off = (issued << 10) + lane * 16;
                if (off < nbytes) d1_dma16(src + off, ring + ((issued & (D1_RING - 1)) << 10));
            }
        };
        for (int j = 0; j < nrows; ++j) {
            const int first = (j * RB) >> 10;
            const int need = ((j + 1) * RB - 1) >> 10;
            const int last = min(need + D1_DEPTH - 1, first + D1_RING - 1);
            asm volatile("" ::: "memory");
            issue_upto(last);
            d1_wait_vm(issued - 1 - need);
            const int o = j * RB;
            float y = 0.0f;
#pragma unroll
            for (int i = 0; i < UPL; ++i) {
                const int G = lane + WAVE * i;
                if (G < NG) {
                    const int bo = o + (G >> 4) * Q2K_BLOCK_BYTES;
                    const uint32_t c = *reinterpret_cast<const uint32_t*>(ring + ((bo + 16 + 4 * (G & 15)) & (D1_RING_BYTES - 1)));
                    const uint32_t sm = ring[(bo + (G & 15)) & (D1_RING_BYTES - 1)];
                    const uint32_t dd = *reinterpret_cast<const uint32_t*>(ring + ((bo + 80) & (D1_RING_BYTES - 1)));
                    if (UP) {
                        const u32x4* xl = reinterpret_cast<const u32x4*>(img);
                        const float2 cs = reinterpret_cast<const float2*>(img + (size_t)NG * 32)[G];
                        const u32x4 lo = xl[G], hi = xl[NG + G];
                        const uint32_t q[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                        y = d1_q2k_group(c, sm, dd, q, cs.x, cs.y, y);
                    } else {
                        const int ri = UP ? 0 : i;
                        y = d1_q2k_group(c, sm, dd, xq[ri], Cg[ri], Sg[ri], y);
                    }
                }
            }
            y = wave_sum(y);
            const int jw = idx + j - r0;
            res.put(jw, y, lane);
            res.maybe_flush(jw, r1 - r0, lane, store);
        }
        idx += nrows;
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Routed rows.  Up pass: operands from the LDS image.  Down pass: operands in
// registers, rebuilt when the wave's rows move on to the next expert.
template <int FMT, bool UP, int UPL>
__device__ void d1_routed(const D1Args& a, int r0, int r1, int lane, const uint8_t* lds) {
    const int NU = FMT == 1 ? a.K / 16 : a.K / 32;
    constexpr int XW = FMT == 1 ? 8 : 16;
    constexpr int RU = UP ? 1 : UPL;         // register operands only in the down pass
    uint32_t xq[RU][XW];
    float Cg[RU], Sg[RU];
    int cur_slot = -1;
    auto stage = [&](int slot) {
#pragma unroll
        for (int i = 0; i < RU; ++i) {
            const int u = lane + WAVE * i;
            if (FMT == 1) {
                if (u < NU) d1_q2k_operands<false>(a, slot, u, xq[i], Cg[i], Sg[i]);
            } else {
#pragma unroll
                for (int c = 0; c < 16; ++c) {
                    const float v0 = u < NU ? d1_act<false>(a, slot, 32 * u + 2 * c, false) : 0.0f;
                    const float v1 = u < NU ? d1_act<false>(a, slot, 32 * u + 2 * c + 1, false) : 0.0f;
                    xq[i][c] = pack_bf16x2(v0, v1);
                }
            }
        }
    };
    D1Results res;
    auto store = [&](int jw, float y) {
        if (UP) a.out_r[r0 + jw] = y;
        else a.eo[r0 + jw] = (uint16_t)f32_to_bf16(y);
    };
    auto compute = [&](const D1Row<FMT, UPL>& b, int idx) {
        if (!UP && b.slot != cur_slot) {     // uniform across the wave
            stage(b.slot);
            cur_slot = b.slot;
        }
        float y = 0.0f;
#pragma unroll
        for (int i = 0; i < UPL; ++i) {
            const int u = lane + WAVE * i;
            if (u < NU) {
                if (UP) {
                    if (FMT == 1) {
                        const u32x4* xl = reinterpret_cast<const u32x4*>(lds);
                        const float2 cs = reinterpret_cast<const float2*>(lds + (size_t)NU * 32)[u];
                        const u32x4 lo = xl[u], hi = xl[NU + u];
                        const uint32_t q[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                        y = d1_q2k_group(b.c[i], b.s[i], b.d[i], q, cs.x, cs.y, y);
                    } else {
                        const u32x4* xl = reinterpret_cast<const u32x4*>(lds);
                        const u32x4 v0 = xl[u], v1 = xl[NU + u], v2 = xl[2 * NU + u], v3 = xl[3 * NU + u];
                        const uint32_t q[16] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3],
                                                v2[0], v2[1], v2[2], v2[3], v3[0], v3[1], v3[2], v3[3]};
                        y = d1_mx_block(b.cw[i], b.s[i], q, y);
                    }
                } else {
                    const int ri = UP ? 0 : i;
                    if (FMT == 1) y = d1_q2k_group(b.c[i], b.s[i], b.d[i], xq[ri], Cg[ri], Sg[ri], y);
                    else y = d1_mx_block(b.cw[i], b.s[i], xq[ri], y);
                }
            }
        }
        y = wave_sum(y);
        res.put(idx - r0, y, lane);
        res.maybe_flush(idx - r0, r1 - r0, lane, store);
    };
    // two named buffers, alternated by a 2-way unrolled loop: the loads of the
    // next row are in flight while the current one is reduced
    D1Row<FMT, UPL> A, B;
    if (r0 >= r1) return;
    d1_load_row(a, r0, lane, A);
    for (int idx = r0; idx < r1; idx += 2) {
        if (idx + 1 < r1) d1_load_row(a, idx + 1, lane, B);
        compute(A, idx);
        if (idx + 1 >= r1) break;
        if (idx + 2 < r1) d1_load_row(a, idx + 2, lane, A);
        compute(B, idx + 1);
    }
}

// Shared-expert rows (bf16 weights).  A row of Ks is cut into ks pieces; lane
// l owns 8-element chunks l, l+64, ... (CPL of them) of a piece.
template <bool UP, int CPL>
__device__ void d1_shared(const D1Args& a, int r0, int r1, int lane, const u32x4* xs) {
    const int piece = a.Ks / a.ks;
    const int NC = piece / 8;
    uint32_t xp[UP ? 1 : CPL][4];         // down pass: h pairs in registers
    int cur_p = -1;
    auto stage = [&](int p) {
        if (UP) return;                      // up pass: x is read from LDS
#pragma unroll
        for (int i = 0; i < (UP ? 1 : CPL); ++i) {
            const int c = lane + WAVE * i;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int col = p * piece + 8 * c + 2 * j;
                const float v0 = c < NC ? d1_act<UP>(a, 0, col, true) : 0.0f;
                const float v1 = c < NC ? d1_act<UP>(a, 0, col + 1, true) : 0.0f;
                xp[i][j] = pack_bf16x2(v0, v1);
            }
        }
    };
    D1Results res;
    auto store = [&](int jw, float y) {     // shared rows in (matrix, row, piece) order
        if (UP) a.out_s[r0 + jw] = y;
        else a.so[r0 + jw] = (uint16_t)f32_to_bf16(y);
    };
    struct Buf { u32x4 wv[CPL]; int p; };
    auto load = [&](Buf& b, int idx) {
        const int per_mat = a.rows_s * a.ks;
        const int mat = idx / per_mat;
        const int rem = idx - mat * per_mat;
        const int r = rem / a.ks;
        b.p = rem - r * a.ks;
        const u32x4* row = reinterpret_cast<const u32x4*>(a.sm[mat] + (size_t)r * a.Ks + (size_t)b.p * piece);
#pragma unroll
        for (int i = 0; i < CPL; ++i) b.wv[i] = row[min(lane + WAVE * i, NC - 1)];   // unconditional
    };
    auto compute = [&](const Buf& b, int idx) {
        if (b.p != cur_p) {
            stage(b.p);
            cur_p = b.p;
        }
        float y = 0.0f;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int c = lane + WAVE * i;
            if (c < NC) {
                uint32_t v[4];
                if (UP) {
                    const u32x4 t = xs[b.p * NC + c];
                    v[0] = t[0]; v[1] = t[1]; v[2] = t[2]; v[3] = t[3];
                } else {
                    const int ri = UP ? 0 : i;
                    v[0] = xp[ri][0]; v[1] = xp[ri][1]; v[2] = xp[ri][2]; v[3] = xp[ri][3];
                }
                y = d1_dot2(b.wv[i][0], v[0], y);
                y = d1_dot2(b.wv[i][1], v[1], y);
                y = d1_dot2(b.wv[i][2], v[2], y);
                y = d1_dot2(b.wv[i][3], v[3], y);
            }
        }
        y = wave_sum(y);
        res.put(idx - r0, y, lane);
        res.maybe_flush(idx - r0, r1 - r0, lane, store);
    };
    Buf A, B;
    if (r0 >= r1) return;
    load(A, r0);
    for (int idx = r0; idx < r1; idx += 2) {
        if (idx + 1 < r1) load(B, idx + 1);
        compute(A, idx);
        if (idx + 1 >= r1) break;
        if (idx + 2 < r1) load(A, idx + 2);
        compute(B, idx + 1);
    }
}

// Chunks per lane of a shared row piece, tied to the routed units per lane
// for the shapes this path takes (shared FFN width == routed FFN width).
template <int FMT, bool UP, int UPL>
struct D1Cpl {
    static constexpr int value = FMT == 1 ? (UP ? UPL : 2 * UPL) : (UP ? 2 * UPL : 4 * UPL);
};

// LDS of a decode1 workgroup: [up-pass image][one Q2K ring per wave].
template <int FMT, bool UP>
__host__ __device__ constexpr size_t d1_ring_offset(int K) {
    return UP ? d1_up_image_bytes<FMT>(K) + (size_t)K * 2 : 0;
}

template <int FMT, bool UP, int UPL>
__global__ __launch_bounds__(256, 2) void decode1_kernel(D1Args a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int lane = threadIdx.x & 63;
    const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int Rr = a.k * a.nmat * a.rows;
    const int Rs = a.rows_s > 0 ? a.nmat * a.rows_s * a.ks : 0;
    if (UP) {
        d1_stage_up_lds<FMT>(a, lds);
        __syncthreads();
    }
    bool shared;
    int r0, r1;
    d1_range(w, a.NW, a.NWs, Rs, Rr, shared, r0, r1);
    if (shared)
        d1_shared<UP, D1Cpl<FMT, UP, UPL>::value>(
            a, r0, r1, lane, reinterpret_cast<const u32x4*>(lds + d1_up_image_bytes<FMT>(a.K)));
    else if (FMT == 1)
        d1_routed_q2k<UP, UPL>(a, r0, r1, lane, lds,
                               lds + d1_ring_offset<FMT, UP>(a.K) + (size_t)(threadIdx.x >> 6) * D1_RING_BYTES);
    else d1_routed<FMT, UP, UPL>(a, r0, r1, lane, lds);
}

// Shared/routed wave split that minimises the largest per-wave byte count:
// start from the byte-proportional split and search its neighbourhood.
static void d1_balance(int NW, long long Rs, double bs, long long Rr, double br, int& NWs) {
    if (Rs == 0) { NWs = 0; return; }
    const double tot_s = Rs * bs, tot_r = Rr * br;
    const int guess = (int)(NW * tot_s / (tot_s + tot_r));
    double best = 1e300;
    NWs = guess < 1 ? 1 : guess;
    for (int s = guess - 32; s <= guess + 32; ++s) {
        if (s < 1 || s >= NW) continue;
        const double x = (double)((Rs + s - 1) / s) * bs;
        const double y = (double)((Rr + (NW - s) - 1) / (NW - s)) * br;
        const double m = x > y ? x : y;
        if (m < best) { best = m; NWs = s; }
    }
}

static int d1_units_per_lane(int fmt, int K) {
    const int unit = fmt == 1 ? 16 : 32;
    return (K / unit + WAVE - 1) / WAVE;
}

bool decode1_supported(const FfnArgs& f) {
    if (f.T != 1) return false;
    if (f.wfmt == 1 && (f.H % 256 || f.F % 256)) return false;     // rows start on a block
    const int uu = d1_units_per_lane(f.wfmt, f.H), ud = d1_units_per_lane(f.wfmt, f.F);
    if (uu > 8 || ud > 8) return false;
    if (f.shared_out && f.Fs > 0) {
        // the shared chunk counts are tied to the routed unit counts
        if (f.Fs != f.F || (f.H / D1_KS_UP) % 8) return false;
        const int cu = ((f.H / D1_KS_UP) / 8 + WAVE - 1) / WAVE, cd = (f.Fs / 8 + WAVE - 1) / WAVE;
        const int eu = f.wfmt == 1 ? uu : 2 * uu, ed = f.wfmt == 1 ? 2 * ud : 4 * ud;
        if (cu > eu || cd > ed) return false;
    }
    return true;
}

size_t decode1_scratch_bytes(int k, int F, int Fs) {
    return ((size_t)k * 2 * F + (size_t)2 * D1_KS_UP * Fs) * 4;
}

template <int FMT, bool UP>
static hipError_t d1_launch(int upl, dim3 grid, size_t lds, hipStream_t s, const D1Args& a) {
    const int stage = UP ? STAGE_FFN_UP : STAGE_FFN_DOWN;
    switch (upl) {
        case 1: return launch_stage(stage, decode1_kernel<FMT, UP, 1>, grid, dim3(256), lds, s, a);
        case 2: return launch_stage(stage, decode1_kernel<FMT, UP, 2>, grid, dim3(256), lds, s, a);
        case 3: return launch_stage(stage, decode1_kernel<FMT, UP, 3>, grid, dim3(256), lds, s, a);
        case 4: return launch_stage(stage, decode1_kernel<FMT, UP, 4>, grid, dim3(256), lds, s, a);
        case 5: return launch_stage(stage, decode1_kernel<FMT, UP, 5>, grid, dim3(256), lds, s, a);
        case 6: return launch_stage(stage, decode1_kernel<FMT, UP, 6>, grid, dim3(256), lds, s, a);
        case 7: return launch_stage(stage, decode1_kernel<FMT, UP, 7>, grid, dim3(256), lds, s, a);
        default: return launch_stage(stage, decode1_kernel<FMT, UP, 8>, grid, dim3(256), lds, s, a);
    }
}

static int g_resident_waves = 0;

static int resident_waves() {
    if (g_resident_waves == 0) {
        int dev = 0, cus = 256;
        if (hipGetDevice(&dev) == hipSuccess) {
            hipDeviceProp_t p;
            if (hipGetDeviceProperties(&p, dev) == hipSuccess && p.multiProcessorCount > 0) cus = p.multiProcessorCount;
        }
        g_resident_waves = cus * 8;     // 2 workgroups of 4 waves per CU (LDS rings + image)
    }
    return g_resident_waves;
}

hipError_t launch_ffn_decode1(const FfnArgs& f, float* scratch, hipStream_t s) {
    const bool shared = f.shared_out != nullptr && f.Fs > 0;
    const int NW = resident_waves();
    float* gu_r = scratch;
    float* gu_s = scratch + (size_t)f.k * 2 * f.F;
    // ---- up: gate and up rows -> fp32 g, u --------------------------------
    {
        D1Args a = {};
        a.K = f.H; a.rows = f.F; a.nmat = 2; a.k = f.k; a.E = f.E;
        a.dstride = expert_data_stride(f.wfmt, f.F, f.H);
        a.sstride = expert_scale_stride(f.F, f.H);
        a.m[0] = f.gate; a.m[1] = f.up; a.sc[0] = f.gate_s; a.sc[1] = f.up_s;
        a.Ks = f.H; a.rows_s = shared ? f.Fs : 0; a.ks = D1_KS_UP;
        a.sm[0] = f.sh_gate; a.sm[1] = f.sh_up;
        a.active = f.active; a.x = reinterpret_cast<const uint16_t*>(f.x);
        a.out_r = gu_r; a.out_s = gu_s;
        a.NW = NW;
        const double br = f.wfmt == 1 ? f.H / 256.0 * 84 : f.H / 2.0 + f.H / 32.0;
        const double bs = 2.0 * f.H / D1_KS_UP;
        d1_balance(NW, shared ? 2LL * f.Fs * D1_KS_UP : 0, bs, 2LL * f.k * f.F, br, a.NWs);
        const int upl = d1_units_per_lane(f.wfmt, f.H);
        const size_t lds = f.wfmt == 1 ? d1_ring_offset<1, true>(f.H) + 4 * (size_t)D1_RING_BYTES
                                       : d1_ring_offset<2, true>(f.H);
        hipError_t e = f.wfmt == 1 ? d1_launch<1, true>(upl, dim3(NW / 4), lds, s, a)
                                   : d1_launch<2, true>(upl, dim3(NW / 4), lds, s, a);
        if (e != hipSuccess) return e;
    }
    // ---- down: h = silu(g) * u, down rows -> expert_out, shared_out --------
    {
        D1Args a = {};
        a.K = f.F; a.rows = f.H; a.nmat = 1; a.k = f.k; a.E = f.E;
        a.dstride = expert_data_stride(f.wfmt, f.H, f.F);
        a.sstride = expert_scale_stride(f.H, f.F);
        a.m[0] = f.down; a.sc[0] = f.down_s;
        a.Ks = f.Fs; a.rows_s = shared ? f.H : 0; a.ks = 1;
        a.sm[0] = f.sh_down;
        a.active = f.active;
        a.gu_r = gu_r; a.gu_s = gu_s;
        a.eo = reinterpret_cast<uint16_t*>(f.expert_out);
        a.so = reinterpret_cast<uint16_t*>(f.shared_out);
        a.NW = NW;
        const double br = f.wfmt == 1 ? f.F / 256.0 * 84 : f.F / 2.0 + f.F / 32.0;
        const double bs = 2.0 * f.Fs;
        d1_balance(NW, shared ? (long long)f.H : 0, bs, (long long)f.k * f.H, br, a.NWs);
        const int upl = d1_units_per_lane(f.wfmt, f.F);
        const size_t lds = f.wfmt == 1 ? 4 * (size_t)D1_RING_BYTES : 0;
        return f.wfmt == 1 ? d1_launch<1, false>(upl, dim3(NW / 4), lds, s, a)
                           : d1_launch<2, false>(upl, dim3(NW / 4), lds, s, a);
    }
}

}  // namespace ds4
