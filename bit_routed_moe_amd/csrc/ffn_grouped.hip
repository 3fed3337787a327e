// Prefill expert FFN (bf16 path): grouped GEMM on the matrix cores.
//
// With thousands of tokens per call every routed expert sees on the order of a
// hundred tokens, so each dequantized weight feeds a hundred multiply-adds and
// the work is a dense contraction: "DS4 分布式Shell客户端" (README mirror,
// section on the distributed prefill) splits prompts into 4096-token chunks,
// and "284B MoEを128GBノートPCに詰め込む" (section on the 790 t/s prefill)
// places the batched-expert work on matrix instructions.  Here it runs on
// gfx950's v_mfma_f32_16x16x32_bf16 with fp32 accumulation.
//
// Work unit: one workgroup (8 waves, two per SIMD) computes a 128-row (up:
// gate + up rows of 128 ffn columns) or 256-row (down) block for one chunk of
// at most 160 tokens of one expert.  A one-workgroup plan kernel lists the chunks
// (experts with more than 160 tokens are split evenly, in 16-token granules).
// With at most 32 tokens (the small-batch layout, two workgroups per CU) the
// shared expert is instead cut into short items of 16 ffn columns or 32
// hidden rows whose reduction range is split over the 8 waves (gg_unit_shs).
//
// Operands, per 16x16x32 MFMA: A = 16 weight rows x 32 reduction columns,
// B = 32 columns x 16 tokens.  Lane l holds row/token (l % 16) and columns
// 8*(l/16) .. +7 of the step.  Each wave owns 2 row tiles (32 rows), so every
// B fragment read from LDS feeds 2 MFMAs, and each weight is dequantized
// exactly once per workgroup, into registers.  Independent VALU work issues
// while the wave's own MFMAs run (a register-only probe: 4 fp32 FMAs per MFMA
// cost nothing on top of the MFMAs); two waves per SIMD also cover each
// other's waits.  Per 128-column stage the lane quarter q (= l/16) owns
// reduction columns 32q .. 32q+31, which is two whole 16-weight Q2K groups
// (one scale byte each), one 32-weight MXFP4 block (one E8M0 scale), or 64
// contiguous bytes of a bf16 row.
//
// Weight decode ("DwarfStar実地分析", section on the intentionally narrow GGUF
// support: the 2-bit routed experts; OCP MX for MXFP4):
//   Q2K   w = RN_bf16(fmaf(d*s, q, -dmin*m)); the 2-bit codes are spread into
//         bytes with masks and converted by v_cvt_pk_f32_fp8 (an fp8 byte
//         0..3 is the subnormal q * 2^-9, so multiplying by d*s*2^9 restores
//         d*s*q exactly).
//   MXFP4 v_cvt_scalef32_pk_bf16_fp4 with the E8M0 scale as fp32 exponent:
//         exact.
//   bf16  (shared expert) loaded as is.
//
// Token rows (x for up, the SwiGLU output h for down) are staged per stage
// into a double-buffered LDS tile by global_load_lds_dwordx4 (1 KiB per wave
// instruction: 4 token rows x 256 B); 16-byte slots are XOR-swizzled by the
// tile row with its 2-bit halves swapped (gg_bswz), the placement under which
// the B reads run without bank conflicts.
//
// Outputs are bf16: h = silu(gate) * up rows [P][F] in sorted pair order
// (shared: [T][Fs]); expert_out [P][H] (shared_out [T][H]).
#include "common.hpp"
#include "formats.hpp"
#include "launch.hpp"

namespace ds4 {

namespace {

constexpr int GG_TT = 16;                     // tokens per MFMA tile
constexpr int GG_NT = 10;                     // token tiles per chunk
constexpr int GG_CT = GG_TT * GG_NT;          // tokens per chunk (160)
constexpr int GG_KS = 128;                    // reduction columns per LDS stage
constexpr int GG_ROWB = GG_KS * 2;            // bytes per staged token row
constexpr int GG_BUF = GG_CT * GG_ROWB;       // one stage buffer: 40 KiB
constexpr int GG_KIND_Q2K = 1, GG_KIND_MX = 2, GG_KIND_BF16 = 3, GG_KIND_Q4K = 4;
constexpr int GG_WAVES = 8;                   // two waves per SIMD
constexpr int GG_RT = 2;                      // 16-row tiles per wave (32 rows)

struct GgChunk {
    int32_t expert;   // routed expert id, or E for the shared expert
    int32_t row0;     // first sorted pair row (routed) or first token (shared)
    int32_t n;        // tokens in the chunk, 1 .. GG_CT
    int32_t pad;
};

constexpr int GG_QUEUES = 8;   // work queues (one per XCD)
constexpr int GG_CTR = 16;     // plan ints [16, 32): work counters of the up and down launches
constexpr int GG_GRID = 256;   // persistent grid: one workgroup per CU

struct GgArgs {
    int E, k, P, T;
    int K, Ks;              // reduction length: routed, shared
    int rows, rows_s;       // rows of one matrix: routed, shared
    int RB;                 // row blocks per chunk in the grid
    int nsh;                // small-batch layout: 1 when chunk 0 is the shared expert's, else 0
    int shs;                // small-batch layout: the shared expert's short items (0: none)
    const GgChunk* chunks;
    const int32_t* n_chunks;
    int32_t* ctr;                  // this launch's GG_QUEUES work counters (zeroed by the plan kernel)
    const int32_t* sorted_pair;
    const uint8_t *w0, *w1;        // routed data: up: gate, up; down: down
    const uint8_t *s0, *s1;        // MXFP4 scales (same roles)
    const uint16_t *sw0, *sw1;     // shared bf16 matrices (same roles)
    const uint16_t* b;             // routed B rows: up x [T][H]; down h [P][F]
    const uint16_t* bs;            // shared B rows: up x [T][H]; down sh_h [T][Fs]
    int ldb, ldbs;                 // their row lengths (elements)
    uint32_t nb, nbs;              // their sizes in bytes (< 2^32)
    uint16_t* out;                 // up: h [P][F]; down: expert_out [P][H]
    uint16_t* outs;                // up: sh_h [T][Fs]; down: shared_out [T][H]
    int ldo, ldos;
    size_t wstride, sstride;       // routed per-expert data / scale strides (bytes)
    // fp8 operands (MXFP4 experts on the scaled matrix instructions)
    const uint8_t* b8;             // routed B rows, E4M3: up xq [T][H]; down h [P][F]
    const uint8_t* bsc;            // their E8M0 scales [rows][K/32]
    uint32_t nb8, nbsc;            // their sizes in bytes
    uint8_t* out8;                 // up: h [P][F] E4M3 codes
    uint8_t* osc;                  // up: h scales [P][F/32]
};

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// ---- chunk plan ----------------------------------------------------------------
// One 1024-thread workgroup: thread e lists the chunks of expert e; the
// shared expert's chunks come first.
__global__ __launch_bounds__(1024) void gg_plan_kernel(const int32_t* __restrict__ offsets, int E, int P, int T,
                                                     int routed, int shared, GgChunk* __restrict__ chunks,
                                                     int32_t* __restrict__ n_chunks, int cmax) {
    __shared__ int tmp[32];
    const int e = threadIdx.x;
    if (e < 2 * GG_QUEUES) n_chunks[GG_CTR + e] = 0;   // the GEMM launches' work counters
    int n = 0, nch = 0;
    if (routed && e < E) {
        const int r0 = offsets[e], r1 = offsets[e + 1];
        n = r1 - r0;
        if (r0 < 0 || r1 > P || n < 0) n = 0;
        nch = ceil_div(n, GG_CT);
    }
    const int nsh = shared ? ceil_div(T, GG_CT) : 0;
    int total;
    const int base = nsh + block_exclusive_scan(nch, tmp, &total);
    total += nsh;
    if (total > cmax) total = 0;   // cannot happen for a valid permutation
    if (total == 0) {
        if (e == 0) n_chunks[0] = 0;
        return;
    }
    auto emit = [&](int c0, int expert, int row0, int cnt, int pieces) {
        const int cs = ceil_div(ceil_div(cnt, pieces), GG_TT) * GG_TT;
        for (int i = 0; i < pieces; ++i) {
            GgChunk c;
            c.expert = expert;
            c.row0 = row0 + i * cs;
            c.n = min(cs, cnt - i * cs);
            c.pad = 0;
            chunks[c0 + i] = c;
        }
    };
    if (nch > 0) emit(base, e, offsets[e], n, nch);
    if (e == 0) {
        if (nsh > 0) emit(0, E, 0, T, nsh);
        n_chunks[0] = total;
    }
}

// ---- LDS DMA -------------------------------------------------------------------
// 64 lanes x 16 B from global memory into LDS at byte address lds_dst +
// 16*lane (LDS addresses are passed as integers computed from the kernel's
// LDS array, never cast back from generic pointers).  Issued as
// inline asm so that the compiler's wait-count pass does not make every later
// LDS read wait for all outstanding loads; the stage loop waits explicitly.
__device__ __forceinline__ void gg_dma16(const void* g, uint32_t lds_dst) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_dst);
    asm volatile(
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, off"
        :
        : "v"(g), "s"(m0)
        : "memory", "m0");
}

__device__ __forceinline__ void gg_wait_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Wait until at most N of this wave's vector-memory operations (loads and LDS
// DMAs, completed in issue order) are outstanding.
template <int N>
__device__ __forceinline__ void gg_wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// The same for a wave-uniform runtime count n in [0, 31] (larger: waits for all).
__device__ __forceinline__ void gg_wait_vm_n(int n) {
    switch (n) {
#define GG_WCASE(k) \
    case k: gg_wait_vm<k>(); break;
        GG_WCASE(0) GG_WCASE(1) GG_WCASE(2) GG_WCASE(3) GG_WCASE(4) GG_WCASE(5) GG_WCASE(6) GG_WCASE(7)
        GG_WCASE(8) GG_WCASE(9) GG_WCASE(10) GG_WCASE(11) GG_WCASE(12) GG_WCASE(13) GG_WCASE(14) GG_WCASE(15)
        GG_WCASE(16) GG_WCASE(17) GG_WCASE(18) GG_WCASE(19) GG_WCASE(20) GG_WCASE(21) GG_WCASE(22) GG_WCASE(23)
        GG_WCASE(24) GG_WCASE(25) GG_WCASE(26) GG_WCASE(27) GG_WCASE(28) GG_WCASE(29) GG_WCASE(30) GG_WCASE(31)
#undef GG_WCASE
        default: gg_wait_all(); break;
    }
}

// ---- LDS carve-up ----------------------------------------------------------------
// [0, 2*GG_BUF): double-buffered token tiles.  After them the raw routed-weight
// bytes, each wave writing and reading only its own 32 rows:
//   Q2K: two buffers of 8 wave regions (32 rows x 96 B + 512 B of slack).
//   A row holds the 16-byte-aligned
//   96-byte window around the 84-byte block that contains the stage's groups
//   (the block starts 0, 4, 8 or 12 bytes in), fetched by buffer_load_dwordx4
//   (6 lanes per row).  When K % 256 == 0 the block holds two stages' groups
//   and is fetched once per two stages; otherwise once per stage.
//   MXFP4: three buffers; per row 4 x 16 B of codes (slot c at
//   c ^ ((row >> 2) & 3)); after the 256 code rows, 64 dwords per
//   (wave, row tile) of which the first 16 hold the tile's E8M0 scale dwords.
// Every DMA here is a buffer load: vector-memory operations of one type
// complete in issue order, which the partial vmcnt waits rely on.
constexpr int GG_QROW = 96;
constexpr int GG_QWAVE = 32 * GG_QROW + 512;   // a wave's 32 rows + room for the idle lanes of its last DMA
constexpr int GG_ABUF_Q2K = GG_WAVES * GG_QWAVE;
constexpr int GG_ABUF_MX = 256 * 64 + GG_WAVES * GG_RT * 64 * 4;
// Token stage buffer for chunks of at most ntm tiles: the staging writes whole
// 32-row tile pairs (the odd tile of an odd count repeats the last token).
constexpr int gg_tbuf(int ntm) { return (ntm + 1) / 2 * 2 * GG_TT * GG_ROWB; }
constexpr int gg_lds_q2k(int ntm) { return 2 * gg_tbuf(ntm) + 2 * GG_ABUF_Q2K; }
constexpr int gg_lds_mx(int ntm) { return 2 * gg_tbuf(ntm) + 3 * GG_ABUF_MX; }
static_assert(gg_tbuf(GG_NT) == GG_BUF, "prefill layout");
// the small-batch layout (chunks of at most 2 tiles) fits two workgroups per CU
static_assert(2 * (gg_lds_q2k(2) + 64) <= 160 * 1024 && 2 * (gg_lds_mx(2) + 64) <= 160 * 1024, "two per CU");

__device__ __forceinline__ int gg_swz(int rr) { return (rr >> 2) & 3; }

// Token rows (256 B = 16 slots of 16 bytes): chunk c of tile row r (0..15)
// sits in slot c ^ gg_bswz(r), the row's two 2-bit halves swapped.  A B
// fragment read (lanes 16q + r read chunk 4q + s of row r, 16 bytes each)
// then takes the minimum 4 LDS cycles per ds_read_b128 on gfx950; the plain
// c ^ r placement measured 8 (a two-way bank conflict).
__device__ __forceinline__ int gg_bswz(int r) { return (r >> 2) | ((r & 3) << 2); }

__device__ __forceinline__ void gg_dma4(const void* g, uint32_t lds_dst) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_dst);
    asm volatile(
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %0, off"
        :
        : "v"(g), "s"(m0)
        : "memory", "m0");
}

// Buffer-resource forms of the LDS DMA: address = base + voffset (per lane,
// 32 bits) + soffset (scalar).  The per-lane offset is checked against the
// resource's byte size (reads past it return zero); the scalar offset is not,
// so every scalar offset used here stays inside its buffer.  A per-lane offset that stays fixed
// across stages plus a scalar stage offset keeps address arithmetic off the
// VALU.  Raw-buffer descriptor for gfx9: stride 0, 32-bit data format.
__device__ __forceinline__ u32x4 gg_rsrc(const void* base, uint32_t bytes) {
    const uint64_t p = reinterpret_cast<uint64_t>(base);
    u32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((uint32_t)p);
    r[1] = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32) & 0xFFFFu);
    r[2] = __builtin_amdgcn_readfirstlane(bytes);
    r[3] = 0x00020000u;
    return r;
}
__device__ __forceinline__ uint32_t gg_m0(uint32_t lds_dst) { return __builtin_amdgcn_readfirstlane(lds_dst); }
__device__ __forceinline__ void gg_bdma4(u32x4 rsrc, uint32_t voff, uint32_t soff, uint32_t lds_dst) {
    asm volatile(
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "buffer_load_dword %0, %1, %2 offen lds"
        :
        : "v"(voff), "s"(rsrc), "s"(soff), "s"(gg_m0(lds_dst))
        : "memory", "m0");
}
__device__ __forceinline__ void gg_bdma16(u32x4 rsrc, uint32_t voff, uint32_t soff, uint32_t lds_dst) {
    asm volatile(
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %0, %1, %2 offen lds"
        :
        : "v"(voff), "s"(rsrc), "s"(soff), "s"(gg_m0(lds_dst))
        : "memory", "m0");
}

template <typename V>
__device__ __forceinline__ V lds_ld(const uint8_t* p) {
    return *reinterpret_cast<const V*>(p);
}

// bf16 shared-expert rows: loaded straight into registers one stage ahead.
struct GgBf16Raw {
    u32x4 v[GG_RT][4];   // [row tile][k-step]
};

__device__ __forceinline__ bf16x8 gg_pack8(const float (&w)[8]) {
    u32x4 v;
    v[0] = pack_bf16x2(w[0], w[1]);
    v[1] = pack_bf16x2(w[2], w[3]);
    v[2] = pack_bf16x2(w[4], w[5]);
    v[3] = pack_bf16x2(w[6], w[7]);
    return __builtin_bit_cast(bf16x8, v);
}

// Decode of the A operands of k-steps 2*gi, 2*gi+1 for one row tile, split
// into an LDS load (issued early) and NS small slices of VALU work that the
// phase loop spreads between matrix instructions (in slice order).  The
// results: r[0] = k-step 2*gi, r[1] = k-step 2*gi+1.
// Pin a value to this point of the instruction stream: an empty volatile asm
// that reads and rewrites it, so the code computing it cannot drift past the
// surrounding scheduling fences (it emits no instruction).
template <typename V>
__device__ __forceinline__ void gg_pin(V& v) {
    asm volatile("" : "+v"(v));
}

template <int KIND>
struct GgDec;

template <>
struct GgDec<GG_KIND_Q2K> {
    static constexpr int NS = 6;
    uint32_t c, scw, dd, x[4];
    float ds9, ndm;
    u32x4 r[2];
    // aux = (offset of the block in the row's window) | (g0 << 8), g0 = the
    // stage's first group in the block (0 or 8)
    __device__ __forceinline__ void load(const uint8_t* ab, int rr, int q4, int gi, int aux) {
        const uint8_t* blk = ab + (rr >> 5) * GG_QWAVE + (rr & 31) * GG_QROW + (aux & 15);
        const int g0 = aux >> 8;
        c = lds_ld<uint32_t>(blk + 16 + 4 * (g0 + 2 * q4 + gi));
        scw = lds_ld<uint32_t>(blk + g0 + 4 * (q4 >> 1));
        dd = lds_ld<uint32_t>(blk + 80);
    }
    // (x[i] holds code 4j + i in byte j; fp8 word 0 of x[i] -> codes (i, i+4),
    // word 1 -> (i+8, i+12); the fp8 byte q is the subnormal q * 2^-9)
    template <int H, int P>
    __device__ __forceinline__ void quad() {
        const auto pa = __builtin_amdgcn_cvt_pk_f32_fp8(x[2 * P], H != 0);
        const auto pb = __builtin_amdgcn_cvt_pk_f32_fp8(x[2 * P + 1], H != 0);
        uint32_t lo = pack_bf16x2(fmaf(ds9, pa[0], ndm), fmaf(ds9, pb[0], ndm));   // codes 8H+2P, +1
        uint32_t hi = pack_bf16x2(fmaf(ds9, pa[1], ndm), fmaf(ds9, pb[1], ndm));   // codes 8H+2P+4, +5
        gg_pin(lo);
        gg_pin(hi);
        r[H][P] = lo;
        r[H][P + 2] = hi;
    }
    template <int J>
    __device__ __forceinline__ void slice(int q4, int gi) {
        if constexpr (J == 0) {
            const uint32_t sc = (scw >> (8 * (2 * (q4 & 1) + gi))) & 0xFFu;
            const float d = half_bits_to_f32(dd & 0xFFFFu);
            const float dmin = half_bits_to_f32(dd >> 16);
            ds9 = d * (float)(sc & 15u) * 512.0f;     // d*s*2^9, exact
            ndm = -(dmin * (float)(sc >> 4));         // -dmin*m, exact
            gg_pin(ds9);
            gg_pin(ndm);
        } else if constexpr (J == 1) {
            const uint32_t M = 0x03030303u;
            x[0] = c & M;
            x[1] = (c >> 2) & M;
            x[2] = (c >> 4) & M;
            x[3] = (c >> 6) & M;
            gg_pin(x[0]);
            gg_pin(x[1]);
            gg_pin(x[2]);
            gg_pin(x[3]);
        } else if constexpr (J == 2) {
            quad<0, 0>();
        } else if constexpr (J == 3) {
            quad<0, 1>();
        } else if constexpr (J == 4) {
            quad<1, 0>();
        } else {
            quad<1, 1>();
        }
    }
};

template <>
struct GgDec<GG_KIND_MX> {
    static constexpr int NS = 3;
    u32x2 cw;
    uint32_t e;
    float scale;
    u32x4 r[2];
    __device__ __forceinline__ void load(const uint8_t* ab, int rr, int q4, int gi, int) {
        cw = lds_ld<u32x2>(ab + rr * 64 + 16 * (q4 ^ gg_swz(rr)) + 8 * gi);
        // scale dword of row rr = 32*w + 16*rt + m at 128*w + 64*rt + m
        e = ab[256 * 64 + (rr + 96 * (rr >> 5) + 48 * ((rr >> 4) & 1)) * 4 + q4];
    }
    template <int J>
    __device__ __forceinline__ void slice(int, int) {
        if constexpr (J == 0) {
            scale = __uint_as_float(e << 23);   // 2^(e-127)
            gg_pin(scale);
        } else {
            const uint32_t c = cw[J - 1];
            uint32_t v0 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, scale, 0));
            uint32_t v1 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, scale, 1));
            uint32_t v2 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, scale, 2));
            uint32_t v3 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, scale, 3));
            gg_pin(v0);
            gg_pin(v1);
            gg_pin(v2);
            gg_pin(v3);
            r[J - 1][0] = v0;
            r[J - 1][1] = v1;
            r[J - 1][2] = v2;
            r[J - 1][3] = v3;
        }
    }
};

// Q4K: codes staged like MXFP4's (64 bytes of a row per stage, 16-byte slot
// c at c ^ ((row >> 2) & 3)); the stage's parameters in the (wave, row tile)
// region after the codes: dword r = s|m bytes of groups 0..3 of the stage
// (of row r of the tile), 16 + r = groups 4..7, 32 + r = d and dmin.  Lane
// quarter q4 decodes groups 2*q4 + gi: nibble q -> byte q (mask) -> fp8 byte
// q, which v_cvt_pk_f32_fp8 turns into q * 2^-9 exactly (codes 0..7 are E4M3
// subnormals, 8..15 the normals (8 + m) * 2^-9); then fmaf(d*s*2^9, ., -dmin*m)
// rounds the weight once and RN gives bf16.
template <>
struct GgDec<GG_KIND_Q4K> {
    static constexpr int NS = 6;
    u32x2 cw;
    uint32_t smw, dd, lo[2], hi[2];
    int g8;
    float ds9, ndm;
    u32x4 r[2];
    __device__ __forceinline__ void load(const uint8_t* ab, int rr, int q4, int gi, int) {
        cw = lds_ld<u32x2>(ab + rr * 64 + 16 * (q4 ^ gg_swz(rr)) + 8 * gi);
        const int pr = 128 * (rr >> 5) + 64 * ((rr >> 4) & 1) + (rr & 15);
        const uint8_t* pb = ab + 256 * 64;
        g8 = 2 * q4 + gi;
        smw = lds_ld<uint32_t>(pb + 4 * (pr + 16 * (g8 >> 2)));
        dd = lds_ld<uint32_t>(pb + 4 * (pr + 32));
    }
    // elements 4P .. 4P+3 of dword H (natural order) -> r[H][2P], r[H][2P+1]
    template <int H, int P>
    __device__ __forceinline__ void quad() {
        const auto pa = __builtin_amdgcn_cvt_pk_f32_fp8(lo[H], P != 0);   // elements 4P, 4P+2
        const auto pb = __builtin_amdgcn_cvt_pk_f32_fp8(hi[H], P != 0);   // elements 4P+1, 4P+3
        uint32_t v0 = pack_bf16x2(fmaf(ds9, pa[0], ndm), fmaf(ds9, pb[0], ndm));
        uint32_t v1 = pack_bf16x2(fmaf(ds9, pa[1], ndm), fmaf(ds9, pb[1], ndm));
        gg_pin(v0);
        gg_pin(v1);
        r[H][2 * P] = v0;
        r[H][2 * P + 1] = v1;
    }
    template <int J>
    __device__ __forceinline__ void slice(int, int) {
        if constexpr (J == 0) {
            const uint32_t sm = (smw >> (8 * (g8 & 3))) & 0xFFu;
            const float d = half_bits_to_f32(dd & 0xFFFFu);
            const float dmin = half_bits_to_f32(dd >> 16);
            ds9 = d * (float)(sm & 15u) * 512.0f;     // d*s*2^9, exact
            ndm = -(dmin * (float)(sm >> 4));         // -dmin*m, exact
            gg_pin(ds9);
            gg_pin(ndm);
        } else if constexpr (J == 1) {
            const uint32_t M = 0x0F0F0F0Fu;
            lo[0] = cw[0] & M;
            hi[0] = (cw[0] >> 4) & M;
            lo[1] = cw[1] & M;
            hi[1] = (cw[1] >> 4) & M;
            gg_pin(lo[0]);
            gg_pin(hi[0]);
            gg_pin(lo[1]);
            gg_pin(hi[1]);
        } else if constexpr (J == 2) {
            quad<0, 0>();
        } else if constexpr (J == 3) {
            quad<0, 1>();
        } else if constexpr (J == 4) {
            quad<1, 0>();
        } else {
            quad<1, 1>();
        }
    }
};

template <int KIND>
__device__ __forceinline__ void gg_slice(GgDec<KIND>& d, int j, int q4, int gi) {
    if constexpr (GgDec<KIND>::NS == 6) {
        switch (j) {
            case 0: d.template slice<0>(q4, gi); break;
            case 1: d.template slice<1>(q4, gi); break;
            case 2: d.template slice<2>(q4, gi); break;
            case 3: d.template slice<3>(q4, gi); break;
            case 4: d.template slice<4>(q4, gi); break;
            default: d.template slice<5>(q4, gi); break;
        }
    } else {
        switch (j) {
            case 0: d.template slice<0>(q4, gi); break;
            case 1: d.template slice<1>(q4, gi); break;
            default: d.template slice<2>(q4, gi); break;
        }
    }
}

// One phase: the MFMAs of k-steps s0, s0+1 for all token tiles (each B
// fragment feeds the wave's GG_RT row tiles), software-pipelined in source
// order: B fragments are read two tile-steps ahead, and when DEC the decode
// slices of the next operands (group gi_dec of the stage staged at ab_dec)
// are spread evenly over the tile-steps, as are the DMA issues for the next
// stages (dma(step, steps)), so the waves do not queue them all at once at
// the top of a stage (PRIO: issued at raised wave priority).  Each step is
// fenced (sched_barrier); within it the compiler orders the MFMAs and the
// VALU share (pinning an MFMA, VALU, MFMA, ... order measured about 1%
// slower); the other wave on the SIMD fills the VALU while this one's MFMAs
// run.
template <int KIND, int NT, bool DEC, bool PRIO, typename DMA>
__device__ __forceinline__ void gg_phase(f32x4 (&acc)[GG_RT][NT], const bf16x8 (&A)[GG_RT][2], const uint8_t* bb,
                                         int q4, int m, int s0, const uint8_t* ab_dec, int rr0, int gi_dec,
                                         const int (&aux)[GG_RT], bf16x8 (&D)[GG_RT][2], const DMA& dma) {
    constexpr int STEPS = 2 * NT;
    constexpr int DK = KIND == GG_KIND_BF16 ? GG_KIND_MX : KIND;
    constexpr int NS = GgDec<DK>::NS;
    constexpr int NSL = GG_RT * NS;                               // slices per phase
    GgDec<DK> dec[GG_RT];
    if constexpr (DEC) {
#pragma unroll
        for (int rt = 0; rt < GG_RT; ++rt) dec[rt].load(ab_dec, rr0 + 16 * rt, q4, gi_dec, aux[rt]);
    }
    auto bread = [&](int i) {
        const int ss = i / NT, t = i % NT;
        const int slot = ((4 * q4 + s0 + ss) ^ gg_bswz(m)) << 4;
        return lds_ld<bf16x8>(bb + t * GG_TT * GG_ROWB + slot);
    };
    bf16x8 b0 = bread(0);
    bf16x8 b1 = STEPS > 1 ? bread(1) : b0;
#pragma unroll
    for (int i = 0; i < STEPS; ++i) {
        bf16x8 b2 = b1;
        if (i + 2 < STEPS) b2 = bread(i + 2);
        const int ss = i / NT, t = i % NT;
#pragma unroll
        for (int rt = 0; rt < GG_RT; ++rt)
            acc[rt][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[rt][ss], b0, acc[rt][t], 0, 0, 0);
        if constexpr (DEC) {
#pragma unroll
            for (int q = 0; q < NSL; ++q)
                if ((q * STEPS) / NSL == i) gg_slice<DK>(dec[q / NS], q % NS, q4, gi_dec);
        }
        if constexpr (PRIO) __builtin_amdgcn_s_setprio(2);
        dma(i, STEPS);   // this step's share of the next stages' DMA issues
        if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_sched_barrier(0);
        b0 = b1;
        b1 = b2;
    }
    if constexpr (DEC) {
#pragma unroll
        for (int rt = 0; rt < GG_RT; ++rt) {
            D[rt][0] = __builtin_bit_cast(bf16x8, dec[rt].r[0]);
            D[rt][1] = __builtin_bit_cast(bf16x8, dec[rt].r[1]);
        }
    }
}

// ---- one work unit ---------------------------------------------------------------
// 8 waves (two per SIMD), each owning GG_RT = 2 row tiles of 16 weight rows:
// up: wave w takes ffn columns f0 = rb*128 + 16*w .. +15, tile 0 from the gate
// matrix and tile 1 from the up matrix (SwiGLU pairs in registers); down:
// rows rb*256 + 32*w .. +31.  Workgroup row rr = 32*w + 16*rt + m.
// NT = token tiles of the chunk (compile time: straight-line tile loops).
// BUF: bytes of one token-row stage buffer (the workgroup's LDS layout).
template <int KIND, bool UP, int NT, int BUF>
__device__ __forceinline__ void gg_unit(const GgArgs& a, const GgChunk& ch, int rb, uint8_t* lds, uint32_t lds32) {
    constexpr bool SH = KIND == GG_KIND_BF16;
    constexpr int ABUF = KIND == GG_KIND_Q2K ? GG_ABUF_Q2K : GG_ABUF_MX;
    static_assert(KIND != GG_KIND_Q4K || GG_ABUF_MX >= 256 * 64 + GG_WAVES * GG_RT * 48 * 4,
                  "a stage's Q4K parameters (48 dwords per wave and row tile) fit the ring buffer");
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int ws = __builtin_amdgcn_readfirstlane(w);
    const int m = lane & 15, q4 = lane >> 4;
    const int K = SH ? a.Ks : a.K;
    // small-batch layout: each step's DMA issues at raised wave priority, so
    // with four waves per SIMD busy on the weight decode the requests still
    // go out at once (16- and 32-token Zipf steps 6% faster; the prefill
    // layout's two waves per SIMD measured 0.5-1% slower with it)
    constexpr bool PRIO = BUF != GG_BUF;
    const int nst = K / GG_KS;
    const int n = ch.n;

    auto wrow = [&](int rt, int mm) { return UP ? rb * 128 + 16 * ws + mm : rb * 256 + 32 * ws + 16 * rt + mm; };
    auto wmat = [&](int rt) -> const uint8_t* {
        if (SH) return reinterpret_cast<const uint8_t*>(UP && rt == 1 ? a.sw1 : a.sw0);
        return (UP && rt == 1 ? a.w1 : a.w0) + (size_t)ch.expert * a.wstride;
    };

    // Raw-weight DMA, each wave for its own 32 rows.  Q2K: instruction j
    // fills WG rows 32*w + 4*j .. +3 (row tile j/4), lane l -> row + (l >> 4),
    // LDS dword slot l & 15 = field (l & 15) ^ (4 * (j & 3)).  MXFP4:
    // instruction j fills rows 32*w + 16*j .. +15, lane l -> row + (l >> 2),
    // slot l & 3 = chunk (l & 3) ^ ((l >> 4) & 3); one dword instruction
    // fetches the wave's 32 scale dwords (lanes 32..63 repeat 0..31 into the
    // wave's padding).
    uint8_t* abase = lds + 2 * BUF;
    const int T16 = K / 16;                      // 16-weight groups per row (a multiple of 8)
    u32x4 ares[2] = {}, sres[2] = {};
    if constexpr (!SH) {
        const uint32_t mbytes = (uint32_t)(KIND == GG_KIND_Q2K ? (size_t)a.rows * K / 256 * 84
                                                              : (size_t)a.rows * K / 2);
        ares[0] = gg_rsrc(wmat(0), mbytes);
        ares[1] = gg_rsrc(wmat(1), mbytes);
        if constexpr (KIND == GG_KIND_MX || KIND == GG_KIND_Q4K) {
            const uint32_t sbytes = (uint32_t)(KIND == GG_KIND_MX ? (size_t)a.rows * K / 32
                                                                  : (size_t)a.rows * K / 256 * 20);
            sres[0] = gg_rsrc((UP ? a.s0 : a.s0) + (size_t)ch.expert * a.sstride, sbytes);
            sres[1] = gg_rsrc((UP ? a.s1 : a.s0) + (size_t)ch.expert * a.sstride, sbytes);
        }
    }
    // Weight DMA number d (0..3) of this wave for stage st (Q2K: the fetch
    // unit starting at stage st, into buffer qbuf; MXFP4: ring buffer st % 3).
    auto issue_a = [&](int st, int qbuf, int d) {
        if constexpr (KIND == GG_KIND_Q2K) {
            // the blocks holding stage st's groups; per row tile 96 lanes (16
            // rows x 6 pieces) in two instructions
            const int rt = d >> 1, b = d & 1;
            const int flat = 64 * b + lane;
            const int rl = flat / 6, piece = flat - 6 * (flat / 6);
            const int64_t fg = (int64_t)wrow(rt, rl < 16 ? rl : 15) * T16 + 8 * min(st, nst - 1);
            const uint32_t vo = (uint32_t)(((fg >> 4) * 84) & ~(int64_t)15) + 16u * (uint32_t)piece;
            // lanes 32..63 of the second instruction (flat >= 96) fetch row 15
            // again into the next tile's first rows (rewritten by that tile's
            // first instruction, issued later and completing in order) or,
            // for the last tile, into the wave region's slack
            const uint32_t dst = lds32 + 2 * BUF + qbuf * GG_ABUF_Q2K + ws * GG_QWAVE + rt * 16 * GG_QROW + b * 1024;
            gg_bdma16(ares[UP && rt == 1 ? 1 : 0], vo, 0u, dst);
        } else if constexpr (KIND == GG_KIND_MX || KIND == GG_KIND_Q4K) {
            const uint32_t ab = lds32 + 2 * BUF + (st % 3) * ABUF;
            const int j = d & 1;
            const int sc = min(st, nst - 1);   // source stage (see issue_x)
            if (KIND == GG_KIND_Q4K && d >= 2) {
                // parameters: lane l -> row l & 15 of tile j, dword l >> 4 of
                // the region: the stage's 8 s|m bytes (record bytes 0..7 for
                // an even stage, 8..15 for an odd one) and d, dmin (16..19);
                // lanes 48..63 repeat d, dmin into the unused dwords
                const int RS = K / 256 * 20;
                const int which = lane >> 4;
                const uint32_t vp = (uint32_t)((lane & 15) * RS + (which < 2 ? 8 * (sc & 1) + 4 * which : 16));
                const uint32_t so = __builtin_amdgcn_readfirstlane((uint32_t)((size_t)wrow(j, 0) * RS + 20 * (sc >> 1)));
                gg_bdma4(sres[UP && j == 1 ? 1 : 0], vp, so, ab + 256 * 64 + (GG_RT * ws + j) * 256);
            } else if (d < 2) {
                const uint32_t vo = (uint32_t)((lane >> 2) * (K / 2) + 16 * ((lane & 3) ^ ((lane >> 4) & 3)));
                const uint32_t so = __builtin_amdgcn_readfirstlane((uint32_t)((size_t)wrow(j, 0) * (K / 2) + 64 * sc));
                gg_bdma16(ares[UP && j == 1 ? 1 : 0], vo, so, ab + (32 * ws + 16 * j) * 64);
            } else {
                // scales: lane l -> row m = l & 15 of tile j (lanes 16..63 repeat)
                const uint32_t vs = (uint32_t)((lane & 15) * (K / 32));
                const uint32_t so = __builtin_amdgcn_readfirstlane((uint32_t)((size_t)wrow(j, 0) * (K / 32) + 4 * sc));
                gg_bdma4(sres[UP && j == 1 ? 1 : 0], vs, so, ab + 256 * 64 + (GG_RT * ws + j) * 256);
            }
        }
    };
    auto stage_a = [&](int st, int qbuf) {
#pragma unroll
        for (int d = 0; d < 4; ++d) issue_a(st, qbuf, d);
    };

    // bf16 rows of the consumer lanes (shared expert)
    const uint8_t* brow[GG_RT];
#pragma unroll
    for (int rt = 0; rt < GG_RT; ++rt) brow[rt] = SH ? wmat(rt) + (size_t)wrow(rt, m) * K * 2 + 64 * q4 : nullptr;
    auto load_bf16 = [&](GgBf16Raw& r, int st) {
#pragma unroll
        for (int rt = 0; rt < GG_RT; ++rt)
#pragma unroll
            for (int s = 0; s < 4; ++s) r.v[rt][s] = *reinterpret_cast<const u32x4*>(brow[rt] + 256 * st + 16 * s);
    };

    // Token rows: instruction i (4 rows of 256 B) goes to wave i % 8; wave w
    // stages tiles t = 2*j + (w >> 2), row r_in = 4*(w & 3) + (lane >> 4) of
    // the tile, 16-byte slot col, from a fixed per-tile byte offset.
    constexpr int NJ = (NT + 1) / 2;
    // DMA j of wave w writes 1 KiB at byte (w + 8 * j) * 1024 of the stage buffer
    static_assert((GG_WAVES - 1 + GG_WAVES * (NJ - 1) + 1) * 1024 <= BUF, "token-row DMAs stay inside a stage buffer");
    // Q2K weight DMA (row tile rt, instruction b) writes 1 KiB at rt * 16 * GG_QROW + b * 1024 of the wave region
    static_assert(KIND != GG_KIND_Q2K || (GG_RT - 1) * 16 * GG_QROW + 2 * 1024 <= GG_QWAVE,
                  "Q2K weight DMAs stay inside the wave's region");
    const int thalf = ws >> 2;
    const int r_in = 4 * (w & 3) + (lane >> 4);
    const int col = (lane & 15) ^ gg_bswz(r_in);
    const u32x4 bres = gg_rsrc(SH ? a.bs : a.b, SH ? a.nbs : a.nb);
    const int ldb = SH ? a.ldbs : a.ldb;
    uint32_t xoff[NJ];
#pragma unroll
    // Rows past the chunk's last token (the last tile's padding, and for odd
    // NT the tile NT that the waves with thalf = 1 also stage: no branch)
    // take an offset past the buffer's range: the buffer load reads nothing
    // there, so those MFMA rows, whose outputs are never stored, do not
    // multiply a copy of real data (prefill 0.4-0.6% faster: the matrix cores
    // draw less power on them, and the clock holds higher)
    for (int j = 0; j < NJ; ++j) {
        int i = 16 * (2 * j + thalf) + r_in;
        const bool pad = i > n - 1;
        if (pad) i = n - 1;
        int r;
        if (UP && !SH) {
            r = a.sorted_pair[ch.row0 + i] / a.k;
            if ((unsigned)r >= (unsigned)a.T) r = 0;   // corrupt permutation: stay in bounds
        } else {
            r = ch.row0 + i;
        }
        xoff[j] = pad ? 0xFFFFFFF0u : (uint32_t)r * (uint32_t)ldb * 2u + 16u * (uint32_t)col;
    }
    auto issue_x = [&](int st, int j) {
        // the source stage is clamped to the last one: the stage loops also
        // request one or two stages past the end (into buffers they no longer
        // read), and the scalar offset is not part of the buffer range check
        gg_bdma16(bres, xoff[j], (uint32_t)min(st, nst - 1) * (GG_KS * 2), lds32 + (st & 1) * BUF + (ws + 8 * j) * 1024);
    };
    auto stage_x = [&](int st) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) issue_x(st, j);
    };

    f32x4 acc[GG_RT][NT];
#pragma unroll
    for (int rt = 0; rt < GG_RT; ++rt)
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[rt][t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    const int rr0 = 32 * w + m;   // + 16*rt: this lane's consumer rows
    if constexpr (SH) {
        GgBf16Raw cur, nxt;
        stage_x(0);
        load_bf16(cur, 0);
        for (int st = 0; st < nst; ++st) {
            gg_wait_all();
            __syncthreads();
            if (st + 1 < nst) {
                stage_x(st + 1);
                load_bf16(nxt, st + 1);
            }
            const uint8_t* bb = lds + (st & 1) * BUF + m * GG_ROWB;
#pragma unroll
            for (int gi = 0; gi < 2; ++gi) {
                bf16x8 A[GG_RT][2], unused[GG_RT][2];
#pragma unroll
                for (int rt = 0; rt < GG_RT; ++rt) {
                    A[rt][0] = __builtin_bit_cast(bf16x8, cur.v[rt][2 * gi]);
                    A[rt][1] = __builtin_bit_cast(bf16x8, cur.v[rt][2 * gi + 1]);
                }
                const int noaux[GG_RT] = {};
                gg_phase<KIND, NT, false, false>(acc, A, bb, q4, m, 2 * gi, nullptr, 0, 0, noaux, unused,
                                          [](int, int) {});
            }
            if (st + 1 < nst) cur = nxt;
        }
    } else {
        // Every stage issues the same DMAs (past the last stage they read
        // bounds-checked addresses into buffers no longer read), so the
        // waits are compile-time counts and the fenced steps hold no branch.
        constexpr int NX = NJ;                                 // token-row DMAs per wave-stage
        constexpr int NA = 2 * GG_RT;                          // weight DMAs per wave and unit
        bf16x8 Ag[GG_RT][2], Ah[GG_RT][2];
        auto first_decode = [&](const uint8_t* ab, const int (&aux)[GG_RT]) {
#pragma unroll
            for (int rt = 0; rt < GG_RT; ++rt) {
                GgDec<KIND> d0;
                d0.load(ab, rr0 + 16 * rt, q4, 0, aux[rt]);
#pragma unroll
                for (int j = 0; j < GgDec<KIND>::NS; ++j) gg_slice<KIND>(d0, j, q4, 0);
                Ag[rt][0] = __builtin_bit_cast(bf16x8, d0.r[0]);
                Ag[rt][1] = __builtin_bit_cast(bf16x8, d0.r[1]);
            }
        };
        // phase DMA schedules: the token rows of stage sx (NX), optionally
        // followed by the weights of unit (au, abuf) (NA)
        auto dma_x_a = [&](int sx, bool with_a, int au, int abuf) {
            return [=, &issue_x, &issue_a](int i, int steps) {
                const int nitems = NX + (with_a ? NA : 0);
#pragma unroll
                for (int j = 0; j < NX; ++j)
                    if ((j * steps) / nitems == i) issue_x(sx, j);
                if (with_a) {
#pragma unroll
                    for (int d = 0; d < NA; ++d)
                        if (((NX + d) * steps) / nitems == i) issue_a(au, abuf, d);
                }
            };
        };
        auto dma_a = [&](int au, int abuf) {
            return [=, &issue_a](int i, int steps) {
#pragma unroll
                for (int d = 0; d < NA; ++d)
                    if ((d * steps) / NA == i) issue_a(au, abuf, d);
            };
        };
        auto dma_none = [](int, int) {};
        if constexpr (KIND == GG_KIND_Q2K) {
            // Raw weights come in fetch units: two stages when K % 256 == 0
            // (unit u = stages 2u, 2u+1, buffer u & 1), else one stage (buffer
            // st & 1).  Phase 0 of stage st runs its k-steps 0,1 on the matrix
            // cores while the VALUs decode its second group; phase 1 runs
            // k-steps 2,3 while they decode the first group of stage st+1 (on
            // the last stage a stale buffer, unused).  Token rows of st+1 are
            // staged during phase 0 and waited for at the end of st; the next
            // unit's weights follow the rows in phase 0 (two-stage units: in an
            // even stage, waited for between the phases of the following odd
            // stage, so they have a stage and a half; one-stage units: waited
            // for between the phases).  A wave's weight buffer holds only its
            // own rows, so the unit can be requested as soon as this wave has
            // decoded the unit before it.
            auto qaux = [&](int st, int (&aux)[GG_RT]) {
#pragma unroll
                for (int rt = 0; rt < GG_RT; ++rt) {
                    const int64_t fg = (int64_t)wrow(rt, m) * T16 + 8 * st;
                    aux[rt] = (int)(((fg >> 4) * 84) & 15) | ((int)(fg & 15) << 8);
                }
            };
            auto abuf_ptr = [&](int buf) { return abase + buf * GG_ABUF_Q2K; };
            stage_x(0);
            stage_a(0, 0);
            gg_wait_all();
            __syncthreads();
            int aux[GG_RT], aux_n[GG_RT];
            qaux(0, aux);
            first_decode(abuf_ptr(0), aux);
            if ((K % 256) == 0) {
                for (int st = 0; st < nst; st += 2) {      // nst is even
                    const int u = st >> 1;
                    // even stage st (unit u), then odd stage st+1 (unit u)
                    {
                        const uint8_t* bb = lds + m * GG_ROWB;                // token buffer 0
                        qaux(st + 1, aux_n);
                        gg_phase<KIND, NT, true, PRIO>(acc, Ag, bb, q4, m, 0, abuf_ptr(u & 1), rr0, 1, aux, Ah,
                                                 dma_x_a(st + 1, true, st + 2, (u + 1) & 1));
                        gg_phase<KIND, NT, true, PRIO>(acc, Ah, bb, q4, m, 2, abuf_ptr(u & 1), rr0, 0, aux_n, Ag,
                                                 dma_none);
                        gg_wait_vm<NA>();                  // token rows of st+1 are in; the next unit may fly
                        __syncthreads();
                    }
                    {
                        const uint8_t* bb = lds + BUF + m * GG_ROWB;       // token buffer 1
                        qaux(st + 2, aux);
                        gg_phase<KIND, NT, true, PRIO>(acc, Ag, bb, q4, m, 0, abuf_ptr(u & 1), rr0, 1, aux_n, Ah,
                                                 dma_x_a(st + 2, false, 0, 0));
                        gg_wait_vm<NX>();                  // the next unit's weights are in
                        gg_phase<KIND, NT, true, PRIO>(acc, Ah, bb, q4, m, 2, abuf_ptr((u + 1) & 1), rr0, 0, aux, Ag,
                                                 dma_none);
                        gg_wait_all();                     // token rows of st+2 are in
                        __syncthreads();
                    }
                }
            } else {
                for (int st = 0; st < nst; ++st) {
                    const uint8_t* bb = lds + (st & 1) * BUF + m * GG_ROWB;
                    qaux(st + 1, aux_n);
                    gg_phase<KIND, NT, true, PRIO>(acc, Ag, bb, q4, m, 0, abuf_ptr(st & 1), rr0, 1, aux, Ah,
                                             dma_x_a(st + 1, true, st + 1, (st + 1) & 1));
                    gg_wait_all();                         // weights (and rows) of st+1 are in
                    gg_phase<KIND, NT, true, PRIO>(acc, Ah, bb, q4, m, 2, abuf_ptr((st + 1) & 1), rr0, 0, aux_n, Ag,
                                             dma_none);
                    __syncthreads();
#pragma unroll
                    for (int rt = 0; rt < GG_RT; ++rt) aux[rt] = aux_n[rt];
                }
            }
        } else {
            // MXFP4: a 3-deep ring of per-stage weight buffers.  During phase 0
            // of stage st the token rows of st+1 and then the weights of st+2
            // are staged; the weights of st+1 (decoded in phase 1) are waited
            // for between the phases, the token rows of st+1 at the end.
            const int noaux[GG_RT] = {};
            stage_x(0);
            stage_a(0, 0);
            stage_a(1, 0);
            gg_wait_vm<NA>();                      // token rows and weights of stage 0 are in
            __syncthreads();
            first_decode(abase, noaux);
            for (int st = 0; st < nst; ++st) {
                const uint8_t* ab = abase + (st % 3) * ABUF;
                const uint8_t* abn = abase + ((st + 1) % 3) * ABUF;
                const uint8_t* bb = lds + (st & 1) * BUF + m * GG_ROWB;
                gg_phase<KIND, NT, true, PRIO>(acc, Ag, bb, q4, m, 0, ab, rr0, 1, noaux, Ah,
                                         dma_x_a(st + 1, true, st + 2, 0));
                gg_wait_vm<NX + NA>();                 // weights of st+1 are in
                gg_phase<KIND, NT, true, PRIO>(acc, Ah, bb, q4, m, 2, abn, rr0, 0, noaux, Ag, dma_none);
                gg_wait_vm<NA>();                      // token rows of st+1 are in
                __syncthreads();
            }
        }
        gg_wait_all();   // no DMA may still target LDS when the workgroup ends
    }

    // epilogue: lane holds rows 4*q4 + i of each row tile for token 16t + m.
    // The output tile is assembled in LDS (the token-row buffers are free
    // once every wave is past the last stage): token row i's 16-byte piece c
    // at i * OCH * 16 + 16 * (c ^ (i & 15)).  Then each row leaves as whole
    // pieces, adjacent lanes on adjacent pieces, instead of 16 scattered
    // 32-byte pieces per store instruction.
    uint16_t* out = SH ? a.outs : a.out;
    const int ldo = SH ? a.ldos : a.ldo;
    constexpr int OCH = UP ? 16 : 32;   // 16-byte pieces per output row (128 or 256 bf16)
    static_assert(NT * GG_TT * OCH * 16 <= 2 * BUF, "the output tile fits the two token-row buffers");
    gg_wait_all();
    __syncthreads();
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int i = 16 * t + m;
        uint8_t* orow = lds + i * (OCH * 16);
        if (UP) {
            u32x2 v;
            v[0] = pack_bf16x2(silu_f32(acc[0][t][0]) * acc[1][t][0], silu_f32(acc[0][t][1]) * acc[1][t][1]);
            v[1] = pack_bf16x2(silu_f32(acc[0][t][2]) * acc[1][t][2], silu_f32(acc[0][t][3]) * acc[1][t][3]);
            const int c = 2 * w + (q4 >> 1);                  // columns 16w + 4q4 .. +3
            *reinterpret_cast<u32x2*>(orow + 16 * (c ^ m) + 8 * (q4 & 1)) = v;
        } else {
#pragma unroll
            for (int rt = 0; rt < GG_RT; ++rt) {
                u32x2 v;
                v[0] = pack_bf16x2(acc[rt][t][0], acc[rt][t][1]);
                v[1] = pack_bf16x2(acc[rt][t][2], acc[rt][t][3]);
                const int c = 4 * w + 2 * rt + (q4 >> 1);     // columns 32w + 16rt + 4q4 .. +3
                *reinterpret_cast<u32x2*>(orow + 16 * (c ^ m) + 8 * (q4 & 1)) = v;
            }
        }
    }
    __syncthreads();
    const int col0 = rb * (UP ? 128 : 256);
    for (int p = threadIdx.x; p < n * OCH; p += GG_WAVES * 64) {
        const int i = p / OCH, c = p % OCH;
        const u32x4 v = lds_ld<u32x4>(lds + i * (OCH * 16) + 16 * (c ^ (i & 15)));
        *reinterpret_cast<u32x4*>(out + (size_t)(ch.row0 + i) * ldo + col0 + 8 * c) = v;
    }
}

// ---- shared expert, small-batch layout ---------------------------------------------
// With at most 32 tokens the shared expert's bf16 rows (4x the bytes of a
// Q2K expert) are streamed rather than computed, and as 128- or 256-row
// blocks a few workgroups streamed 3.7 MB each long after the routed blocks
// were done.  Here a work item is 16 ffn columns (up: 16 gate + 16 up rows)
// or 32 hidden rows (down), the item's 8 waves split its reduction range in
// 128-column groups, and each wave loads its weight rows and token rows
// straight into registers (no staging, no barrier in the loop): four MFMA
// steps of requests in flight, each step's registers reloaded for the next
// group as soon as its MFMAs have read them.  The 8 partial sums meet in LDS
// once.  Within a group, lane quarter q holds columns 32q + 8s .. +7 at step
// s, for the weights and the tokens alike (the same column order on both
// operands).
template <bool UP, int NT>
__device__ __forceinline__ void gg_unit_shs(const GgArgs& a, const GgChunk& ch, int item, uint8_t* lds) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int m = lane & 15, q4 = lane >> 4;
    const int K = a.Ks;
    const int ng = K / GG_KS;
    const int g0 = (w * ng) / GG_WAVES, g1 = ((w + 1) * ng) / GG_WAVES;   // this wave's groups
    const int n = ch.n;
    const uint16_t* wr[GG_RT];
#pragma unroll
    for (int rt = 0; rt < GG_RT; ++rt) {
        const int row = UP ? 16 * item + m : 32 * item + 16 * rt + m;
        wr[rt] = (UP && rt == 1 ? a.sw1 : a.sw0) + (size_t)row * K + 32 * q4;
    }
    const uint16_t* xr[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int i = min(16 * t + m, n - 1);   // padding lanes repeat the last token
        xr[t] = a.bs + (size_t)(ch.row0 + i) * a.ldbs + 32 * q4;
    }
    f32x4 acc[GG_RT][NT];
#pragma unroll
    for (int rt = 0; rt < GG_RT; ++rt)
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[rt][t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    if (g1 > g0) {
        u32x4 A[4][GG_RT], B[4][NT];
        // step s of group g (past the wave's last group: that group again,
        // into registers no longer read)
        auto load = [&](int g, int s) {
            const int col = min(g, g1 - 1) * GG_KS + 8 * s;
#pragma unroll
            for (int rt = 0; rt < GG_RT; ++rt) A[s][rt] = *reinterpret_cast<const u32x4*>(wr[rt] + col);
#pragma unroll
            for (int t = 0; t < NT; ++t) B[s][t] = *reinterpret_cast<const u32x4*>(xr[t] + col);
        };
#pragma unroll
        for (int s = 0; s < 4; ++s) load(g0, s);
        for (int g = g0; g < g1; ++g) {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
#pragma unroll
                for (int t = 0; t < NT; ++t)
#pragma unroll
                    for (int rt = 0; rt < GG_RT; ++rt)
                        acc[rt][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8, A[s][rt]), __builtin_bit_cast(bf16x8, B[s][t]), acc[rt][t], 0,
                            0, 0);
                load(g + 1, s);
            }
        }
    }
    // partial sums: wave w's tile (rt, t) at float (((rt * NT + t) * 8 + w) * 64 + lane) * 4
    static_assert(GG_RT * NT * GG_WAVES * 64 * 16 <= gg_lds_q2k(2) && GG_RT * NT * GG_WAVES * 64 * 16 <= gg_lds_mx(2),
                  "the partial sums fit the small-batch layout's LDS");
    float* part = reinterpret_cast<float*>(lds);
#pragma unroll
    for (int rt = 0; rt < GG_RT; ++rt)
#pragma unroll
        for (int t = 0; t < NT; ++t)
            *reinterpret_cast<f32x4*>(part + (((rt * NT + t) * GG_WAVES + w) * 64 + lane) * 4) = acc[rt][t];
    __syncthreads();
    // thread o sums tile (rt, t) of lane l over the waves: up pairs the gate
    // and up tiles of (t, l) in one thread
    constexpr int NOUT = (UP ? 1 : GG_RT) * NT * 64;
    const int o = threadIdx.x;
    if (o < NOUT) {
        const int l = o & 63, t = (o >> 6) % NT, rt = UP ? 0 : (o >> 6) / NT;
        const int i = 16 * t + (l & 15);
        auto sum = [&](int r) {
            f32x4 v = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int ww = 0; ww < GG_WAVES; ++ww)
                v += *reinterpret_cast<const f32x4*>(part + (((r * NT + t) * GG_WAVES + ww) * 64 + l) * 4);
            return v;
        };
        if (i < n) {
            uint16_t* orow = a.outs + (size_t)(ch.row0 + i) * a.ldos;
            u32x2 v;
            if (UP) {
                const f32x4 g = sum(0), u = sum(1);
                v[0] = pack_bf16x2(silu_f32(g[0]) * u[0], silu_f32(g[1]) * u[1]);
                v[1] = pack_bf16x2(silu_f32(g[2]) * u[2], silu_f32(g[3]) * u[3]);
                *reinterpret_cast<u32x2*>(orow + 16 * item + 4 * (l >> 4)) = v;
            } else {
                const f32x4 y = sum(rt);
                v[0] = pack_bf16x2(y[0], y[1]);
                v[1] = pack_bf16x2(y[2], y[3]);
                *reinterpret_cast<u32x2*>(orow + 32 * item + 16 * rt + 4 * (l >> 4)) = v;
            }
        }
    }
}

// ---- MXFP4 weights x MXFP8 tokens on the scaled matrix instructions ---------
// v_mfma_scale_f32_16x16x128_f8f6f4, A = 16 weight rows x 128 reduction
// columns in E2M1, B = 128 columns x 16 tokens in E4M3, each with one E8M0
// scale per 32 columns, fp32 accumulation.  Operand layout on gfx950 (found
// with single-element probes): lane l holds A row l%16, columns 32(l/16) ..
// +31 as 16 bytes in natural nibble order, with A's scale for (row l%16, block
// l/16); B token l%16, columns 16(l/16) .. +15 in bytes 0..15 and columns
// 64 + 16(l/16) .. +15 in bytes 16..31, with B's scale for (token l%16, block
// l/16); D as for the bf16 instruction.  A lane's A operand is thus 16
// contiguous bytes of a weight row and its scale the row's own E8M0 byte: the
// weights go to the matrix cores without any decode.
//
// One stage = 128 reduction columns = one instruction per (row tile, token
// tile).  LDS: a 4-deep ring of weight buffers (the MXFP4 layout above: weights
// are fetched three stages ahead), and 3-deep rings of token rows (160 rows x
// 128 B; 16-byte slot s of row r at s ^ ((r >> 1) & 7), so the 16 lanes of a B
// read with one lane quarter hit 16 distinct bank groups) and of token scales
// (the stage's 4 scale bytes of chunk row i as the dword at 256*(i/32) +
// 4*(i%32)), fetched two stages ahead.
// (rows written by the token DMAs: whole 64-row groups, (2 * NT + 7) / 8 of them)
constexpr int GG8_TBUF = (2 * GG_NT + 7) / 8 * 64 * 128;
static_assert(GG8_TBUF >= GG_CT * 128, "a chunk's token rows fit");
constexpr int GG8_SBUF = GG_WAVES * 256;
constexpr int GG8_NA = 4;   // weight DMAs per wave-stage (2 code rows-blocks, 2 scale dwords)
constexpr int GG_LDS_MX8 = 3 * GG8_TBUF + 3 * GG8_SBUF + 4 * GG_ABUF_MX;
static_assert(GG_LDS_MX8 >= 2 * GG_BUF, "the shared expert's bf16 tiles fit in the same LDS");
static_assert(GG_LDS_MX8 + 64 <= 160 * 1024, "LDS of one workgroup");

typedef int v8i __attribute__((ext_vector_type(8)));

// NT = token tiles of the chunk.  Waves and rows as in gg_unit.  The up
// projection's epilogue quantizes h = silu(gate) * up to MXFP8 right away: a
// 32-column block spans the 16 columns of two neighbouring waves, whose block
// maxima meet in LDS.
template <bool UP, int NT>
__device__ __forceinline__ void gg_unit_mx8(const GgArgs& a, const GgChunk& ch, int rb, uint8_t* lds,
                                            uint32_t lds32) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int ws = __builtin_amdgcn_readfirstlane(w);
    const int m = lane & 15, q4 = lane >> 4;
    const int K = a.K;
    const int nst = K / 128;
    const int n = ch.n;
    const uint8_t* const tbase = lds;
    const uint8_t* const sbase = lds + 3 * GG8_TBUF;
    const uint8_t* const abase = sbase + 3 * GG8_SBUF;
    const uint32_t sb32 = lds32 + 3 * GG8_TBUF, ab32 = sb32 + 3 * GG8_SBUF;

    // weights: the MXFP4 fetch of gg_unit, one stage = 128 columns, ring slot st & 3
    auto wrow0 = [&](int j) { return UP ? rb * 128 + 16 * ws : rb * 256 + 32 * ws + 16 * j; };
    const size_t eoff = (size_t)ch.expert * a.wstride, esoff = (size_t)ch.expert * a.sstride;
    const uint32_t mbytes = (uint32_t)((size_t)a.rows * K / 2), sbytes = (uint32_t)((size_t)a.rows * K / 32);
    const u32x4 ares[2] = {gg_rsrc(a.w0 + eoff, mbytes), gg_rsrc((UP ? a.w1 : a.w0) + eoff, mbytes)};
    const u32x4 sres[2] = {gg_rsrc(a.s0 + esoff, sbytes), gg_rsrc((UP ? a.s1 : a.s0) + esoff, sbytes)};
    const uint32_t avo = (uint32_t)((lane >> 2) * (K / 2) + 16 * ((lane & 3) ^ ((lane >> 4) & 3)));
    const uint32_t avs = (uint32_t)((lane & 15) * (K / 32));
    auto issue_a = [&](int st, int d) {
        const uint32_t ab = ab32 + (st & 3) * GG_ABUF_MX;
        const int j = d & 1;
        if (d < 2) {
            const uint32_t so = __builtin_amdgcn_readfirstlane((uint32_t)(wrow0(j) * (K / 2) + 64 * min(st, nst - 1)));
            gg_bdma16(ares[UP && j == 1 ? 1 : 0], avo, so, ab + (32 * ws + 16 * j) * 64);
        } else {
            const uint32_t so = __builtin_amdgcn_readfirstlane((uint32_t)(wrow0(j) * (K / 32) + 4 * min(st, nst - 1)));
            gg_bdma4(sres[UP && j == 1 ? 1 : 0], avs, so, ab + 256 * 64 + (GG_RT * ws + j) * 256);
        }
    };

    // token rows: DMA j of wave w stages chunk rows 8*(w + 8j) .. +7 (lane l ->
    // row + (l >> 3), LDS slot l & 7); rows past the chunk repeat its last token
    constexpr int NX = (2 * NT + 7) / 8;
    // the last DMA (w = 7, j = NX - 1) ends 1 KiB past byte 8 * (7 + 8 * (NX - 1)) * 128
    static_assert((8 * (GG_WAVES - 1 + GG_WAVES * (NX - 1)) + 8) * 128 <= GG8_TBUF,
                  "a stage's token-row DMAs stay inside their ring buffer");
    static_assert(GG_WAVES * 256 <= GG8_SBUF, "a stage's token-scale DMAs stay inside their ring buffer");
    auto tok_row = [&](int i) {
        if (i > n - 1) i = n - 1;
        int r;
        if (UP) {
            r = a.sorted_pair[ch.row0 + i] / a.k;
            if ((unsigned)r >= (unsigned)a.T) r = 0;   // corrupt permutation: stay in bounds
        } else {
            r = ch.row0 + i;
        }
        return r;
    };
    const u32x4 bres = gg_rsrc(a.b8, a.nb8);
    const u32x4 bsres = gg_rsrc(a.bsc, a.nbsc);
    uint32_t xoff[NX];
#pragma unroll
    for (int j = 0; j < NX; ++j) {
        const int rl = 8 * (ws + 8 * j) + (lane >> 3);
        const int slot = (lane & 7) ^ ((rl >> 1) & 7);
        xoff[j] = (uint32_t)tok_row(rl) * (uint32_t)K + 16u * (uint32_t)slot;
    }
    const uint32_t soff = (uint32_t)tok_row(32 * ws + (lane & 31)) * (uint32_t)(K / 32);
    auto issue_x = [&](int st, int j) {
        gg_bdma16(bres, xoff[j], (uint32_t)min(st, nst - 1) * 128u, lds32 + (st % 3) * GG8_TBUF + 8 * (ws + 8 * j) * 128);
    };
    // lanes 32..63 repeat 0..31 into the upper half of the wave's 256 bytes
    auto issue_s = [&](int st) {
        gg_bdma4(bsres, soff, (uint32_t)min(st, nst - 1) * 4u, sb32 + (st % 3) * GG8_SBUF + 256 * ws);
    };
    constexpr int NXB = NX + 1;
    auto issue_stage = [&](int stx, int sta) {   // in the order the waits assume
#pragma unroll
        for (int j = 0; j < NX; ++j) issue_x(stx, j);
        issue_s(stx);
#pragma unroll
        for (int d = 0; d < GG8_NA; ++d) issue_a(sta, d);
    };

    f32x4 acc[GG_RT][NT];
#pragma unroll
    for (int rt = 0; rt < GG_RT; ++rt)
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[rt][t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // In flight at the end of stage st: the weights of st+2, and the token rows
    // and scales of st+2 with the weights of st+3 (issued during st).  Every
    // stage issues the same DMAs (past the last stage they read bounds-checked
    // addresses into buffers no longer read), so the wait is a constant.
    constexpr int AHEAD = 2 * GG8_NA + NXB;
#pragma unroll
    for (int d = 0; d < GG8_NA; ++d) issue_a(0, d);
    issue_stage(0, 1);
    issue_stage(1, 2);
    gg_wait_vm<AHEAD>();
    __syncthreads();

    const int rr0 = 32 * w + m;
    const int bsw = (m >> 1) & 7;
    for (int st = 0; st < nst; ++st) {
        const uint8_t* ab = abase + (st & 3) * GG_ABUF_MX;
        const uint8_t* tb = tbase + (st % 3) * GG8_TBUF + m * 128;
        const uint8_t* sb = sbase + (st % 3) * GG8_SBUF;
        v8i A[GG_RT];
        int sa[GG_RT];
#pragma unroll
        for (int rt = 0; rt < GG_RT; ++rt) {
            const int rr = rr0 + 16 * rt;
            const u32x4 c = lds_ld<u32x4>(ab + rr * 64 + 16 * (q4 ^ gg_swz(rr)));
            A[rt] = v8i{(int)c[0], (int)c[1], (int)c[2], (int)c[3], 0, 0, 0, 0};
            sa[rt] = ab[256 * 64 + (rr + 96 * (rr >> 5) + 48 * ((rr >> 4) & 1)) * 4 + q4];
        }
        auto bread = [&](int t, v8i& b, int& sc) {
            const uint8_t* row = tb + t * 16 * 128;
            const u32x4 lo = lds_ld<u32x4>(row + 16 * (q4 ^ bsw));
            const u32x4 hi = lds_ld<u32x4>(row + 16 * ((4 + q4) ^ bsw));
            b = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
            const int i = 16 * t + m;
            sc = sb[256 * (i >> 5) + 4 * (i & 31) + q4];
        };
        v8i b0, b1, b2;
        int s0, s1, s2;
        bread(0, b0, s0);
        if (NT > 1) bread(1, b1, s1);
        constexpr int ITEMS = NXB + GG8_NA;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            if (t + 2 < NT) bread(t + 2, b2, s2);
#pragma unroll
            for (int rt = 0; rt < GG_RT; ++rt)
                acc[rt][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[rt], b0, acc[rt][t], 4, 0, 0, sa[rt],
                                                                               0, s0);
            // this step's share of the DMAs for stages st+2 (tokens) and st+3 (weights)
#pragma unroll
            for (int q = 0; q < ITEMS; ++q) {
                if ((q * NT) / ITEMS == t) {
                    if (q < NX) issue_x(st + 2, q);
                    else if (q == NX) issue_s(st + 2);
                    else issue_a(st + 3, q - NXB);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            b0 = b1;
            s0 = s1;
            b1 = b2;
            s1 = s2;
        }
        gg_wait_vm<AHEAD>();   // tokens of st+1 and weights of st+1 are in
        __syncthreads();
    }
    gg_wait_all();   // no DMA may still target LDS when the unit ends

    if constexpr (UP) {
        // h = silu(gate) * up, then MXFP8 per 32 columns: this wave's 16
        // columns of a token are 4 lanes (q4) x 4 values; the block's other 16
        // belong to wave w ^ 1
        __syncthreads();   // every wave's DMAs have landed: the token buffers are free
        float* xa = reinterpret_cast<float*>(lds);
        float am[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            float mx = 0.0f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float v = silu_f32(acc[0][t][j]) * acc[1][t][j];
                acc[0][t][j] = v;
                mx = fmaxf(mx, fabsf(v));
            }
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            am[t] = mx;
            if (q4 == 0) xa[(w * NT + t) * 16 + m] = mx;
        }
        __syncthreads();
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const float amax = fmaxf(am[t], xa[((w ^ 1) * NT + t) * 16 + m]);
            const uint32_t sbyte = mx8_scale_byte(amax);
            const float inv = mx8_inv_scale(sbyte);
            const int i = 16 * t + m;
            if (i < n) {
                const size_t row = (size_t)(ch.row0 + i);
                const int c0 = rb * 128 + 16 * w;
                *reinterpret_cast<uint32_t*>(a.out8 + row * a.ldo + c0 + 4 * q4) =
                    mx8_pack4(acc[0][t][0] * inv, acc[0][t][1] * inv, acc[0][t][2] * inv, acc[0][t][3] * inv);
                if (q4 == 0 && (w & 1) == 0) a.osc[row * (a.ldo / 32) + c0 / 32] = (uint8_t)sbyte;
            }
        }
    } else {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int i = 16 * t + m;
            if (i < n) {
                uint16_t* orow = a.out + (size_t)(ch.row0 + i) * a.ldo;
#pragma unroll
                for (int rt = 0; rt < GG_RT; ++rt) {
                    u32x2 v;
                    v[0] = pack_bf16x2(acc[rt][t][0], acc[rt][t][1]);
                    v[1] = pack_bf16x2(acc[rt][t][2], acc[rt][t][3]);
                    *reinterpret_cast<u32x2*>(orow + rb * 256 + 32 * w + 16 * rt + 4 * q4) = v;
                }
            }
        }
    }
}

template <bool UP>
__device__ __forceinline__ void gg_dispatch_mx8(const GgArgs& a, const GgChunk& ch, int rb, uint8_t* lds,
                                                uint32_t lds32, int nt) {
    switch (nt) {
        case 1: gg_unit_mx8<UP, 1>(a, ch, rb, lds, lds32); break;
        case 2: gg_unit_mx8<UP, 2>(a, ch, rb, lds, lds32); break;
        case 3: gg_unit_mx8<UP, 3>(a, ch, rb, lds, lds32); break;
        case 4: gg_unit_mx8<UP, 4>(a, ch, rb, lds, lds32); break;
        case 5: gg_unit_mx8<UP, 5>(a, ch, rb, lds, lds32); break;
        case 6: gg_unit_mx8<UP, 6>(a, ch, rb, lds, lds32); break;
        case 7: gg_unit_mx8<UP, 7>(a, ch, rb, lds, lds32); break;
        case 8: gg_unit_mx8<UP, 8>(a, ch, rb, lds, lds32); break;
        case 9: gg_unit_mx8<UP, 9>(a, ch, rb, lds, lds32); break;
        default: gg_unit_mx8<UP, 10>(a, ch, rb, lds, lds32); break;
    }
}

// NTM: the most token tiles a chunk of this launch holds (GG_NT, or 2 for the
// small-batch layout); nt <= NTM.
template <int KIND, bool UP, int NTM>
__device__ __forceinline__ void gg_dispatch(const GgArgs& a, const GgChunk& ch, int rb, uint8_t* lds, uint32_t lds32,
                                            int nt) {
    constexpr int B = gg_tbuf(NTM);
    if constexpr (NTM == 2) {
        if (nt == 1) gg_unit<KIND, UP, 1, B>(a, ch, rb, lds, lds32);
        else gg_unit<KIND, UP, 2, B>(a, ch, rb, lds, lds32);
    } else {
        switch (nt) {
            case 1: gg_unit<KIND, UP, 1, B>(a, ch, rb, lds, lds32); break;
            case 2: gg_unit<KIND, UP, 2, B>(a, ch, rb, lds, lds32); break;
            case 3: gg_unit<KIND, UP, 3, B>(a, ch, rb, lds, lds32); break;
            case 4: gg_unit<KIND, UP, 4, B>(a, ch, rb, lds, lds32); break;
            case 5: gg_unit<KIND, UP, 5, B>(a, ch, rb, lds, lds32); break;
            case 6: gg_unit<KIND, UP, 6, B>(a, ch, rb, lds, lds32); break;
            case 7: gg_unit<KIND, UP, 7, B>(a, ch, rb, lds, lds32); break;
            case 8: gg_unit<KIND, UP, 8, B>(a, ch, rb, lds, lds32); break;
            case 9: gg_unit<KIND, UP, 9, B>(a, ch, rb, lds, lds32); break;
            default: gg_unit<KIND, UP, 10, B>(a, ch, rb, lds, lds32); break;
        }
    }
}

// Grid: RB row blocks x (chunks padded to a multiple of 8).  The hardware
// deals workgroups to the 8 XCDs round-robin, so workgroup b runs on XCD b % 8;
// chunk c is placed on XCD c % 8 and its RB row blocks are dealt to that XCD
// back to back: they share the chunk's token rows in the XCD's L2.
template <int FMT, bool UP, int NTM>
__global__ __launch_bounds__(GG_WAVES * 64, NTM == GG_NT ? 1 : 4) void gg_kernel(GgArgs a) {
    // FMT 1 Q2K, 2 MXFP4, 4 Q4K; 3: MXFP4 routed experts on fp8 operands
    // (prefill layout only)
    static_assert(FMT != 3 || NTM == GG_NT, "fp8 operands use the prefill layout");
    __shared__ __attribute__((aligned(1024))) uint8_t lds[FMT == 1 ? gg_lds_q2k(NTM)
                                                           : ((FMT == 2 || FMT == 4) ? gg_lds_mx(NTM) : GG_LDS_MX8)];
    __shared__ int s_item;
    const uint32_t lds32 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds;
    // Work queue q = blockIdx % 8 (the XCD the workgroup runs on) holds the
    // (chunk, row block) items of chunks q, q+8, ..., row blocks of a chunk
    // adjacent, so one chunk's token rows stay in one L2.  Workgroups take
    // items in order from their queue's counter until it runs past the end.
    // With the prefill layout they then take items from the other queues in
    // turn (the counters are device-scope atomics), so no XCD idles while
    // another still has items (about 1% on 1024-4096 tokens).  The short
    // small-batch launches do not: 512 workgroups polling the other seven
    // counters at the end cost more than the balance gains (7-13% slower).
    // In the small-batch layout the shared expert's chunk (chunk 0 when
    // a.nsh = 1) is not dealt as row blocks: its a.shs short items follow the
    // routed items of every queue, item s in queue s % 8.
    const int q0 = blockIdx.x & (GG_QUEUES - 1);
    const int nc = a.n_chunks[0];
    const int c0 = NTM == GG_NT ? 0 : a.nsh;   // first chunk dealt as row blocks
    for (int qi = 0; qi < (NTM == GG_NT ? GG_QUEUES : 1); ++qi) {
        const int q = (q0 + qi) & (GG_QUEUES - 1);
        const int nri = (nc - c0 > q ? (nc - c0 - q + GG_QUEUES - 1) / GG_QUEUES : 0) * a.RB;
        const int nsi = NTM != GG_NT && a.shs > q ? (a.shs - q + GG_QUEUES - 1) / GG_QUEUES : 0;
        const int items = nri + nsi;
        if (items == 0) continue;
        for (;;) {
            if (threadIdx.x == 0) s_item = atomicAdd(a.ctr + q, 1);
            __syncthreads();
            const int j = __builtin_amdgcn_readfirstlane(s_item);   // uniform: scalar registers
            __syncthreads();
            if (j >= items) break;
            if constexpr (NTM != GG_NT) {
                if (j >= nri) {
                    const int si = (j - nri) * GG_QUEUES + q;
                    const GgChunk ch = a.chunks[0];
                    if (ch.expert != a.E || ch.row0 != 0 || ch.n < 1 || ch.n > a.T || ch.n > NTM * GG_TT) continue;
                    if (ch.n > GG_TT)
                        gg_unit_shs<UP, 2>(a, ch, si, lds);
                    else
                        gg_unit_shs<UP, 1>(a, ch, si, lds);
                    continue;
                }
            }
            const int chunk = c0 + (j / a.RB) * GG_QUEUES + q;
            const int rb = j % a.RB;
            const GgChunk ch = a.chunks[chunk];
            const bool shared = ch.expert == a.E;
            if (ch.n < 1 || ch.n > NTM * GG_TT || ch.row0 < 0 || (!shared && (ch.expert < 0 || ch.expert > a.E)))
                continue;
            if (ch.row0 + ch.n > (shared ? a.T : a.P)) continue;
            const int rows = shared ? a.rows_s : a.rows;
            if ((rb + 1) * (UP ? 128 : 256) > rows) continue;
            const int nt = (ch.n + GG_TT - 1) / GG_TT;
            if (shared) {
                // (the small-batch layout takes the shared expert as short items only)
                if constexpr (NTM == GG_NT) gg_dispatch<GG_KIND_BF16, UP, NTM>(a, ch, rb, lds, lds32, nt);
            } else if constexpr (FMT == 3)
                gg_dispatch_mx8<UP>(a, ch, rb, lds, lds32, nt);
            else
                gg_dispatch<FMT, UP, NTM>(a, ch, rb, lds, lds32, nt);
        }
    }
}

int gg_max_chunks(int E, int P, int T, bool routed, bool shared) {
    int c = 0;
    if (routed) c += (E < P ? E : P) + P / GG_CT + 1;
    if (shared) c += (T + GG_CT - 1) / GG_CT;
    return c;
}

template <int FMT, bool UP>
hipError_t gg_launch(const FfnArgs& f, const GgChunk* chunks, const int32_t* n_chunks, int cmax, bool routed,
                     bool shared, hipStream_t s) {
    GgArgs a;
    a.E = f.E;
    a.k = f.k;
    a.T = f.T;
    a.P = f.T * f.k;
    a.K = UP ? f.H : f.F;
    a.Ks = UP ? f.H : f.Fs;
    a.rows = UP ? f.F : f.H;
    a.rows_s = UP ? f.Fs : f.H;
    // Persistent grid, a multiple of the queue count: one workgroup per CU with
    // the prefill layout; two per CU with the small-batch layout (at most 32
    // tokens, so every chunk has at most 2 tiles), twice the weight bytes in
    // flight where the few token tiles leave the matrix cores idle.
    const bool small = FMT != 3 && f.T <= 2 * GG_TT;
    const int rbr = routed ? (UP ? f.F / 128 : f.H / 256) : 0;
    const int rbs = shared && !small ? (UP ? f.Fs / 128 : f.H / 256) : 0;
    a.RB = rbr > rbs ? rbr : rbs;
    // small-batch layout: the shared expert as short items (16 ffn columns for
    // up, 32 hidden rows for down), chunk 0 of the plan
    a.nsh = shared && small ? 1 : 0;
    a.shs = shared && small ? (UP ? f.Fs / 16 : f.H / 32) : 0;
    a.chunks = chunks;
    a.n_chunks = n_chunks;
    a.sorted_pair = f.sorted_pair;
    a.w0 = UP ? f.gate : f.down;
    a.w1 = UP ? f.up : nullptr;
    a.s0 = UP ? f.gate_s : f.down_s;
    a.s1 = UP ? f.up_s : nullptr;
    a.sw0 = UP ? f.sh_gate : f.sh_down;
    a.sw1 = UP ? f.sh_up : nullptr;
    a.b = UP ? static_cast<const uint16_t*>(f.x) : static_cast<const uint16_t*>(f.h);
    a.bs = UP ? static_cast<const uint16_t*>(f.x) : static_cast<const uint16_t*>(f.sh_h);
    a.ldb = UP ? f.H : f.F;
    a.ldbs = UP ? f.H : f.Fs;
    a.nb = (uint32_t)((UP ? (size_t)f.T * f.H : (size_t)f.T * f.k * f.F) * 2);
    a.nbs = (uint32_t)((UP ? (size_t)f.T * f.H : (size_t)f.T * f.Fs) * 2);
    a.out = UP ? static_cast<uint16_t*>(f.h) : static_cast<uint16_t*>(f.expert_out);
    a.outs = UP ? static_cast<uint16_t*>(f.sh_h) : static_cast<uint16_t*>(f.shared_out);
    a.ldo = UP ? f.F : f.H;
    a.ldos = UP ? f.Fs : f.H;
    const int wf = FMT == 3 ? WFMT_MX : FMT;
    a.wstride = expert_data_stride(wf, UP ? f.F : f.H, UP ? f.H : f.F);
    a.sstride = expert_scale_stride(wf, UP ? f.F : f.H, UP ? f.H : f.F);
    if (FMT == 3) {
        const size_t P = (size_t)f.T * f.k;
        a.b8 = UP ? f.xq : static_cast<const uint8_t*>(f.h);
        a.bsc = UP ? f.xsc : f.hsc;
        a.nb8 = (uint32_t)(UP ? (size_t)f.T * f.H : P * f.F);
        a.nbsc = (uint32_t)(UP ? (size_t)f.T * f.H / 32 : P * f.F / 32);
        a.out8 = UP ? static_cast<uint8_t*>(f.h) : nullptr;
        a.osc = UP ? f.hsc : nullptr;
    } else {
        a.b8 = nullptr;
        a.bsc = nullptr;
        a.nb8 = a.nbsc = 0;
        a.out8 = nullptr;
        a.osc = nullptr;
    }
    const int gmax = small ? 2 * GG_GRID : GG_GRID;
    const int cpad = (cmax + GG_QUEUES - 1) / GG_QUEUES * GG_QUEUES;
    const long long most = (long long)cpad * a.RB + a.shs;
    if (most == 0) return hipSuccess;
    const int grid = most < gmax ? (int)((most + GG_QUEUES - 1) / GG_QUEUES * GG_QUEUES) : gmax;
    a.ctr = const_cast<int32_t*>(n_chunks) + GG_CTR + (UP ? 0 : GG_QUEUES);
    const int stage = UP ? STAGE_FFN_UP : STAGE_FFN_DOWN;
    if constexpr (FMT != 3) {
        if (small) return launch_stage(stage, gg_kernel<FMT, UP, 2>, dim3(grid), dim3(GG_WAVES * 64), 0, s, a);
    }
    return launch_stage(stage, gg_kernel<FMT, UP, GG_NT>, dim3(grid), dim3(GG_WAVES * 64), 0, s, a);
}

}  // namespace

size_t grouped_plan_bytes(int E, int T, int k, bool shared) {
    const long long P = (long long)T * k;
    const int c = gg_max_chunks(E, (int)P, T, true, shared);
    return 256 + (size_t)c * sizeof(GgChunk);
}

bool grouped_supports_q4k() { return true; }

bool grouped_supported(const FfnArgs& f) {
    // token-row sources are addressed with 32-bit buffer offsets
    const size_t lim = (size_t)1 << 32;
    return (size_t)f.T * f.H * 2 < lim && (size_t)f.T * f.k * f.F * 2 < lim && (size_t)f.T * f.Fs * 2 < lim;
}

hipError_t launch_grouped_plan(const FfnArgs& f, bool routed, bool shared, hipStream_t s) {
    const int P = f.T * f.k;
    const int cmax = gg_max_chunks(f.E, P, f.T, routed, shared);
    int32_t* n_chunks = f.plan;
    GgChunk* chunks = reinterpret_cast<GgChunk*>(reinterpret_cast<uint8_t*>(f.plan) + 256);
    hipLaunchKernelGGL(gg_plan_kernel, dim3(1), dim3(1024), 0, s, f.offsets, f.E, P, f.T, routed ? 1 : 0,
                       shared ? 1 : 0, chunks, n_chunks, cmax);
    return hipGetLastError();
}

hipError_t launch_grouped_gemm(const FfnArgs& f, bool routed, bool shared, hipStream_t s) {
    if (!routed && !shared) return hipSuccess;
    if (!grouped_supported(f)) return hipErrorInvalidValue;
    const int P = f.T * f.k;
    const int cmax = gg_max_chunks(f.E, P, f.T, routed, shared);
    const int32_t* n_chunks = f.plan;
    const GgChunk* chunks = reinterpret_cast<const GgChunk*>(reinterpret_cast<const uint8_t*>(f.plan) + 256);
    hipError_t e;
    if (f.wfmt == 2 && f.mx8) {
        e = gg_launch<3, true>(f, chunks, n_chunks, cmax, routed, shared, s);
        return e != hipSuccess ? e : gg_launch<3, false>(f, chunks, n_chunks, cmax, routed, shared, s);
    }
    if (f.wfmt == 1) {
        e = gg_launch<1, true>(f, chunks, n_chunks, cmax, routed, shared, s);
        return e != hipSuccess ? e : gg_launch<1, false>(f, chunks, n_chunks, cmax, routed, shared, s);
    }
    if (f.wfmt == WFMT_Q4K) {
        e = gg_launch<4, true>(f, chunks, n_chunks, cmax, routed, shared, s);
        return e != hipSuccess ? e : gg_launch<4, false>(f, chunks, n_chunks, cmax, routed, shared, s);
    }
    e = gg_launch<2, true>(f, chunks, n_chunks, cmax, routed, shared, s);
    return e != hipSuccess ? e : gg_launch<2, false>(f, chunks, n_chunks, cmax, routed, shared, s);
}

hipError_t launch_ffn_grouped_bf16(const FfnArgs& f, bool routed, bool shared, hipStream_t s) {
    if (!routed && !shared) return hipSuccess;
    if (!grouped_supported(f)) return hipErrorInvalidValue;
    const hipError_t e = launch_grouped_plan(f, routed, shared, s);
    if (e != hipSuccess) return e;
    return launch_grouped_gemm(f, routed, shared, s);
}

}  // namespace ds4
