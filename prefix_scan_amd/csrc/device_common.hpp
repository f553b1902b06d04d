// device_common.hpp -- wave64 primitives, tile I/O and the chained-carry
// (decoupled look-back) state shared by the libscan kernels on gfx950.
//
// Tiles.  A kernel sees its array through a "virtual" index v = i + head,
// where head = (address / 4) mod 4 moves the array's first element to the
// slot it occupies inside its 16-byte granule.  Virtual slot 4q .. 4q+3 is
// then one aligned 16-byte chunk, so every thread moves whole chunks with
// dwordx4 loads and stores.  Valid elements are the virtual range [vlo, vhi).
// A tile of BLOCK threads x V chunks is laid out chunk-major: chunk k of
// thread `tid` is virtual chunk (tile_start / 4) + k * BLOCK + tid, so each
// wave instruction moves 1 KiB of contiguous memory.  Element order inside a
// tile is (k, tid, j), j the element inside the chunk.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace libscan {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ uint32_t lane_id()
{
    return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

// Mask of the lanes below this one.
__device__ __forceinline__ uint64_t lanemask_lt()
{
    const uint32_t l = lane_id();
    return l == 0 ? 0ull : (~0ull >> (64 - l));
}

__device__ __forceinline__ uint64_t ballot(bool p)
{
    return __builtin_amdgcn_ballot_w64(p);
}

// ---------------------------------------------------------------------------
// DPP wave scans.  row_shr:1,2,4,8 scan each row of 16 lanes (a lane whose
// source falls outside its row reads 0); row_bcast:15 then adds lane 15's
// total into row 1 and lane 47's into row 3; row_bcast:31 adds lane 31's
// total into rows 2 and 3.
// ---------------------------------------------------------------------------
constexpr int kDppRowShr1 = 0x111;
constexpr int kDppRowShr2 = 0x112;
constexpr int kDppRowShr4 = 0x114;
constexpr int kDppRowShr8 = 0x118;
constexpr int kDppWaveShr1 = 0x138;
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp(uint32_t x)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROW_MASK, 0xF, false);
}

// Inclusive wave scan under wrapping u32 add.
__device__ __forceinline__ uint32_t wave_incl_add(uint32_t x)
{
    x += dpp<kDppRowShr1, 0xF>(x);
    x += dpp<kDppRowShr2, 0xF>(x);
    x += dpp<kDppRowShr4, 0xF>(x);
    x += dpp<kDppRowShr8, 0xF>(x);
    x += dpp<kDppRowBcast15, 0xA>(x);
    x += dpp<kDppRowBcast31, 0xC>(x);
    return x;
}

__device__ __forceinline__ uint32_t wave_bcast_last(uint32_t x)
{
    return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

// Wave-wide sum, the same in every lane.
__device__ __forceinline__ uint32_t wave_sum(uint32_t x)
{
    return wave_bcast_last(wave_incl_add(x));
}

// The previous lane's value (0 in lane 0).
__device__ __forceinline__ uint32_t wave_shr1(uint32_t x)
{
    return dpp<kDppWaveShr1, 0xF>(x);
}

// ---------------------------------------------------------------------------
// The integer operators of a scan or reduction (CAIRN "Concurrency",
// "reduce and compact"): add_wrap, mul_wrap, &, |, ^, min and max on
// 32-bit values, each with its identity; min and max compare as unsigned,
// or as signed (MinS, MaxS).  All are associative and commutative, so any
// grouping gives the same bits.
// ---------------------------------------------------------------------------
struct OpAdd {
    static constexpr uint32_t identity = 0u;
    __device__ static __forceinline__ uint32_t apply(uint32_t a, uint32_t b) { return a + b; }
};
struct OpMul {
    static constexpr uint32_t identity = 1u;
    __device__ static __forceinline__ uint32_t apply(uint32_t a, uint32_t b) { return a * b; }
};
struct OpAnd {
    static constexpr uint32_t identity = 0xFFFFFFFFu;
    __device__ static __forceinline__ uint32_t apply(uint32_t a, uint32_t b) { return a & b; }
};
struct OpOr {
    static constexpr uint32_t identity = 0u;
    __device__ static __forceinline__ uint32_t apply(uint32_t a, uint32_t b) { return a | b; }
};
struct OpXor {
    static constexpr uint32_t identity = 0u;
    __device__ static __forceinline__ uint32_t apply(uint32_t a, uint32_t b) { return a ^ b; }
};
struct OpMin {
    static constexpr uint32_t identity = 0xFFFFFFFFu;
    __device__ static __forceinline__ uint32_t apply(uint32_t a, uint32_t b) { return a < b ? a : b; }
};
struct OpMax {
    static constexpr uint32_t identity = 0u;
    __device__ static __forceinline__ uint32_t apply(uint32_t a, uint32_t b) { return a > b ? a : b; }
};
// min and max of the words read as two's-complement int32.
struct OpMinS {
    static constexpr uint32_t identity = 0x7FFFFFFFu;
    __device__ static __forceinline__ uint32_t apply(uint32_t a, uint32_t b)
    {
        return (int32_t)a < (int32_t)b ? a : b;
    }
};
struct OpMaxS {
    static constexpr uint32_t identity = 0x80000000u;
    __device__ static __forceinline__ uint32_t apply(uint32_t a, uint32_t b)
    {
        return (int32_t)a > (int32_t)b ? a : b;
    }
};

// The same operators on unsigned 64-bit values (CAIRN writes its rows as
// u64), each with its identity mod 2^64.
struct OpAdd64 {
    static constexpr uint64_t identity = 0u;
    __device__ static __forceinline__ uint64_t apply(uint64_t a, uint64_t b) { return a + b; }
};
struct OpMul64 {
    static constexpr uint64_t identity = 1u;
    __device__ static __forceinline__ uint64_t apply(uint64_t a, uint64_t b) { return a * b; }
};
struct OpAnd64 {
    static constexpr uint64_t identity = ~0ull;
    __device__ static __forceinline__ uint64_t apply(uint64_t a, uint64_t b) { return a & b; }
};
struct OpOr64 {
    static constexpr uint64_t identity = 0u;
    __device__ static __forceinline__ uint64_t apply(uint64_t a, uint64_t b) { return a | b; }
};
struct OpXor64 {
    static constexpr uint64_t identity = 0u;
    __device__ static __forceinline__ uint64_t apply(uint64_t a, uint64_t b) { return a ^ b; }
};
struct OpMin64 {
    static constexpr uint64_t identity = ~0ull;
    __device__ static __forceinline__ uint64_t apply(uint64_t a, uint64_t b) { return a < b ? a : b; }
};
struct OpMax64 {
    static constexpr uint64_t identity = 0u;
    __device__ static __forceinline__ uint64_t apply(uint64_t a, uint64_t b) { return a > b ? a : b; }
};
struct OpMinS64 {
    static constexpr uint64_t identity = 0x7FFFFFFFFFFFFFFFull;
    __device__ static __forceinline__ uint64_t apply(uint64_t a, uint64_t b)
    {
        return (int64_t)a < (int64_t)b ? a : b;
    }
};
struct OpMaxS64 {
    static constexpr uint64_t identity = 0x8000000000000000ull;
    __device__ static __forceinline__ uint64_t apply(uint64_t a, uint64_t b)
    {
        return (int64_t)a > (int64_t)b ? a : b;
    }
};

// DPP move whose disabled lanes (source outside the row, masked rows) read
// `old` -- the operator's identity.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_or(uint32_t x, uint32_t old)
{
    return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)x, CTRL, ROW_MASK, 0xF, false);
}

// Operators whose identity is not 0 take their DPP steps as | or unsigned
// max on the words XORed with a mask: a & b = ~(~a | ~b), min(a, b) =
// ~max(~a, ~b), and flipping the sign bit maps signed order onto unsigned
// order (flipping the other 31 bits too reverses it).  The mask maps 0 to
// the operator's identity.  Under identity 0 each step is one DPP
// instruction whose disabled lanes read 0 (bound_ctrl), with no register
// holding the identity; & otherwise takes a DPP move and a separate and per
// step, and the scans of &, min and signed min and max spilled.
template <class Op>
struct DppFlip {
    using Base = Op;
    static constexpr uint32_t mask = 0u;
};
template <>
struct DppFlip<OpAnd> {
    using Base = OpOr;
    static constexpr uint32_t mask = 0xFFFFFFFFu;
};
template <>
struct DppFlip<OpMin> {
    using Base = OpMax;
    static constexpr uint32_t mask = 0xFFFFFFFFu;
};
template <>
struct DppFlip<OpMinS> {
    using Base = OpMax;
    static constexpr uint32_t mask = 0x7FFFFFFFu;
};
template <>
struct DppFlip<OpMaxS> {
    using Base = OpMax;
    static constexpr uint32_t mask = 0x80000000u;
};

// x XOR Op's flip mask, opaque to the compiler: it would otherwise fold the
// flips into the steps between them (& would turn back into & steps).
template <class Op>
__device__ __forceinline__ uint32_t dpp_flip(uint32_t x)
{
    constexpr uint32_t kMask = DppFlip<Op>::mask;
    uint32_t y;
    if constexpr (kMask == 0xFFFFFFFFu)
        asm("v_not_b32 %0, %1" : "=v"(y) : "v"(x));
    else
        asm("v_xor_b32 %0, %2, %1" : "=v"(y) : "v"(x), "n"(kMask));
    return y;
}

// Inclusive wave scan under Op (the same steps as wave_incl_add).
template <class Op>
__device__ __forceinline__ uint32_t wave_incl(uint32_t x)
{
    constexpr uint32_t kFlip = DppFlip<Op>::mask;
    if constexpr (__is_same(Op, OpAdd)) {
        return wave_incl_add(x);
    } else if constexpr (kFlip != 0u) {
        static_assert((kFlip ^ DppFlip<Op>::Base::identity) == Op::identity, "mask maps identities");
        return dpp_flip<Op>(wave_incl<typename DppFlip<Op>::Base>(dpp_flip<Op>(x)));
    } else {
        constexpr uint32_t e = Op::identity;
        x = Op::apply(x, dpp_or<kDppRowShr1, 0xF>(x, e));
        x = Op::apply(x, dpp_or<kDppRowShr2, 0xF>(x, e));
        x = Op::apply(x, dpp_or<kDppRowShr4, 0xF>(x, e));
        x = Op::apply(x, dpp_or<kDppRowShr8, 0xF>(x, e));
        x = Op::apply(x, dpp_or<kDppRowBcast15, 0xA>(x, e));
        x = Op::apply(x, dpp_or<kDppRowBcast31, 0xC>(x, e));
        return x;
    }
}

// The fold of the whole wave under Op, in every lane.
template <class Op>
__device__ __forceinline__ uint32_t wave_fold(uint32_t x)
{
    return wave_bcast_last(wave_incl<Op>(x));
}

// The previous lane's value (Op's identity in lane 0).
template <class Op>
__device__ __forceinline__ uint32_t wave_shr1_op(uint32_t x)
{
    constexpr uint32_t kFlip = DppFlip<Op>::mask;
    if constexpr (kFlip != 0u)
        return dpp_flip<Op>(dpp_or<kDppWaveShr1, 0xF>(dpp_flip<Op>(x), 0u));
    else
        return dpp_or<kDppWaveShr1, 0xF>(x, Op::identity);
}

// 64-bit lanes: each DPP step moves the two halves with the same control,
// so a lane always receives one whole value (or the identity's halves).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint64_t dpp64_or(uint64_t x, uint64_t old)
{
    const uint32_t lo = dpp_or<CTRL, ROW_MASK>((uint32_t)x, (uint32_t)old);
    const uint32_t hi = dpp_or<CTRL, ROW_MASK>((uint32_t)(x >> 32), (uint32_t)(old >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// Inclusive wave scan of u64 values under Op (the steps of wave_incl_add),
// keeping operand order: lane l ends with x_0 op x_1 op .. op x_l, so Op
// need not commute (the segmented pair of segflags_kernels.hip does not).
// Inclusive wave scan of u64 values under wrapping add: each step one
// carry-chained pair of DPP adds (low word, then high word with the carry).
// Lanes whose source lies outside the row, or in a masked row, are disabled
// for both instructions of the step and keep their value (x + 0).  Each step
// starts with two wait states, which a DPP read of a VGPR written by the
// instruction before it needs.
#define LIBSCAN_DPP64_STEP(CTRL, RMASK)                                              \
    "s_nop 1\n"                                                                      \
    "v_add_co_u32_dpp %0, vcc, %0, %0 " CTRL " row_mask:" RMASK " bank_mask:0xf\n"    \
    "v_addc_co_u32_dpp %1, vcc, %1, %1, vcc " CTRL " row_mask:" RMASK " bank_mask:0xf\n"
__device__ __forceinline__ uint64_t wave_incl64_add(uint64_t x)
{
    uint32_t lo = (uint32_t)x, hi = (uint32_t)(x >> 32);
    asm(LIBSCAN_DPP64_STEP("row_shr:1", "0xf")
                 LIBSCAN_DPP64_STEP("row_shr:2", "0xf")
                 LIBSCAN_DPP64_STEP("row_shr:4", "0xf")
                 LIBSCAN_DPP64_STEP("row_shr:8", "0xf")
                 LIBSCAN_DPP64_STEP("row_bcast:15", "0xa")
                 LIBSCAN_DPP64_STEP("row_bcast:31", "0xc")
                 "s_nop 1\n"
                 : "+v"(lo), "+v"(hi)
                 :
                 : "vcc");
    return ((uint64_t)hi << 32) | lo;
}
#undef LIBSCAN_DPP64_STEP

// Two such scans interleaved step by step: each step's four instructions
// put three others between every DPP read and the write of its register in
// the step before, more than the two wait states it needs, so only the first
// step waits.
#define LIBSCAN_DPP64_STEP2(CTRL, RMASK)                                             \
    "v_add_co_u32_dpp %0, vcc, %0, %0 " CTRL " row_mask:" RMASK " bank_mask:0xf\n"    \
    "v_addc_co_u32_dpp %1, vcc, %1, %1, vcc " CTRL " row_mask:" RMASK " bank_mask:0xf\n" \
    "v_add_co_u32_dpp %2, vcc, %2, %2 " CTRL " row_mask:" RMASK " bank_mask:0xf\n"    \
    "v_addc_co_u32_dpp %3, vcc, %3, %3, vcc " CTRL " row_mask:" RMASK " bank_mask:0xf\n"
__device__ __forceinline__ void wave_incl64_add2(uint64_t &a, uint64_t &b)
{
    uint32_t alo = (uint32_t)a, ahi = (uint32_t)(a >> 32);
    uint32_t blo = (uint32_t)b, bhi = (uint32_t)(b >> 32);
    asm("s_nop 1\n"
        LIBSCAN_DPP64_STEP2("row_shr:1", "0xf")
        LIBSCAN_DPP64_STEP2("row_shr:2", "0xf")
        LIBSCAN_DPP64_STEP2("row_shr:4", "0xf")
        LIBSCAN_DPP64_STEP2("row_shr:8", "0xf")
        LIBSCAN_DPP64_STEP2("row_bcast:15", "0xa")
        LIBSCAN_DPP64_STEP2("row_bcast:31", "0xc")
        "s_nop 1\n"
        : "+v"(alo), "+v"(ahi), "+v"(blo), "+v"(bhi)
        :
        : "vcc");
    a = ((uint64_t)ahi << 32) | alo;
    b = ((uint64_t)bhi << 32) | blo;
}
#undef LIBSCAN_DPP64_STEP2

// Two inclusive wave scans of u64 values under unsigned max, step by step.
// A step compares each lane with its source lane by a DPP subtract-with-
// borrow pair (source - own; the final borrow, in VCC, says own is larger)
// and keeps own or takes the source's halves with two DPP selects: four
// instructions a step, against five that first move the source's halves
// into registers.  The subtraction's result is dropped.  Lanes whose source
// lies outside the row, or in a masked row, are disabled for all four
// instructions and keep their value.  The two scans' steps alternate, so
// each DPP read follows the write of its register by four instructions.
#define LIBSCAN_MAX64_STEP(LO, HI, CTRL, RMASK)                                                    \
    "v_sub_co_u32_dpp %4, vcc, " LO ", " LO " " CTRL " row_mask:" RMASK " bank_mask:0xf\n"       \
    "v_subb_co_u32_dpp %4, vcc, " HI ", " HI ", vcc " CTRL " row_mask:" RMASK " bank_mask:0xf\n" \
    "v_cndmask_b32_dpp " LO ", " LO ", " LO ", vcc " CTRL " row_mask:" RMASK " bank_mask:0xf\n"  \
    "v_cndmask_b32_dpp " HI ", " HI ", " HI ", vcc " CTRL " row_mask:" RMASK " bank_mask:0xf\n"
#define LIBSCAN_MAX64_STEP2(CTRL, RMASK)                                                            \
    LIBSCAN_MAX64_STEP("%0", "%1", CTRL, RMASK)                                                    \
    LIBSCAN_MAX64_STEP("%2", "%3", CTRL, RMASK)
__device__ __forceinline__ void wave_incl64_max2(uint64_t &a, uint64_t &b)
{
    uint32_t alo = (uint32_t)a, ahi = (uint32_t)(a >> 32);
    uint32_t blo = (uint32_t)b, bhi = (uint32_t)(b >> 32);
    uint32_t t;
    asm("s_nop 1\n"
        LIBSCAN_MAX64_STEP2("row_shr:1", "0xf")
        LIBSCAN_MAX64_STEP2("row_shr:2", "0xf")
        LIBSCAN_MAX64_STEP2("row_shr:4", "0xf")
        LIBSCAN_MAX64_STEP2("row_shr:8", "0xf")
        LIBSCAN_MAX64_STEP2("row_bcast:15", "0xa")
        LIBSCAN_MAX64_STEP2("row_bcast:31", "0xc")
        "s_nop 1\n"
        : "+v"(alo), "+v"(ahi), "+v"(blo), "+v"(bhi), "=&v"(t)
        :
        : "vcc");
    a = ((uint64_t)ahi << 32) | alo;
    b = ((uint64_t)bhi << 32) | blo;
}
#undef LIBSCAN_MAX64_STEP2
#undef LIBSCAN_MAX64_STEP

// The min / max family of u64 operators as unsigned max of flipped values:
// x ^ mask reverses the order for min (all bits), maps the signed order to
// the unsigned one for signed max (the sign bit), and does both for signed
// min (all bits but the sign).
template <class Op>
struct MaxFlip64 {
    static constexpr bool is = false;
};
template <>
struct MaxFlip64<OpMax64> {
    static constexpr bool is = true;
    static constexpr uint64_t mask = 0ull;
};
template <>
struct MaxFlip64<OpMin64> {
    static constexpr bool is = true;
    static constexpr uint64_t mask = ~0ull;
};
template <>
struct MaxFlip64<OpMaxS64> {
    static constexpr bool is = true;
    static constexpr uint64_t mask = 0x8000000000000000ull;
};
template <>
struct MaxFlip64<OpMinS64> {
    static constexpr bool is = true;
    static constexpr uint64_t mask = 0x7FFFFFFFFFFFFFFFull;
};

template <class Op>
__device__ __forceinline__ uint64_t wave_incl64(uint64_t x)
{
    if constexpr (__is_same(Op, OpAdd64))
        return wave_incl64_add(x);
    constexpr uint64_t e = Op::identity;
    x = Op::apply(dpp64_or<kDppRowShr1, 0xF>(x, e), x);
    x = Op::apply(dpp64_or<kDppRowShr2, 0xF>(x, e), x);
    x = Op::apply(dpp64_or<kDppRowShr4, 0xF>(x, e), x);
    x = Op::apply(dpp64_or<kDppRowShr8, 0xF>(x, e), x);
    x = Op::apply(dpp64_or<kDppRowBcast15, 0xA>(x, e), x);
    x = Op::apply(dpp64_or<kDppRowBcast31, 0xC>(x, e), x);
    return x;
}

// One DPP move of a u64 lane value whose identity under Op is the source
// of lanes outside the row (or in a row not written).  When the identity is
// 0 and every row is written, bound_ctrl makes out-of-row lanes read 0
// directly, so the move needs no copy of the identity in its destination.
template <int CTRL, int ROW_MASK, uint64_t ID>
__device__ __forceinline__ uint64_t dpp64_id(uint64_t x)
{
    if constexpr (ID == 0 && ROW_MASK == 0xF) {
        const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)x, CTRL, 0xF, 0xF, true);
        const uint32_t hi =
            (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(x >> 32), CTRL, 0xF, 0xF, true);
        return ((uint64_t)hi << 32) | lo;
    } else {
        return dpp64_or<CTRL, ROW_MASK>(x, ID);
    }
}

// Two inclusive wave scans of u64 values under Op, step by step together:
// each step's DPP reads of one scan follow the other scan's writes, so
// neither waits for the register it reads (the steps of wave_incl64).
template <class Op>
__device__ __forceinline__ void wave_incl64_pair(uint64_t &a, uint64_t &b)
{
    constexpr uint64_t e = Op::identity;
#define LIBSCAN_PAIR_STEP(CTRL, RMASK)                                                             \
    {                                                                                              \
        const uint64_t pa = dpp64_id<CTRL, RMASK, e>(a);                                           \
        const uint64_t pb = dpp64_id<CTRL, RMASK, e>(b);                                           \
        a = Op::apply(pa, a);                                                                      \
        b = Op::apply(pb, b);                                                                      \
    }
    LIBSCAN_PAIR_STEP(kDppRowShr1, 0xF)
    LIBSCAN_PAIR_STEP(kDppRowShr2, 0xF)
    LIBSCAN_PAIR_STEP(kDppRowShr4, 0xF)
    LIBSCAN_PAIR_STEP(kDppRowShr8, 0xF)
    LIBSCAN_PAIR_STEP(kDppRowBcast15, 0xA)
    LIBSCAN_PAIR_STEP(kDppRowBcast31, 0xC)
#undef LIBSCAN_PAIR_STEP
}

// Inclusive wave scans of V values under Op, two at a time -- but for the
// 64-bit multiply, whose steps are long enough to need no partner and whose
// pairs only add register pressure (5.7% slower paired).
template <class Op, int V>
__device__ __forceinline__ void wave_incl64_n(const uint64_t (&e)[V], uint64_t (&w)[V])
{
    if constexpr (__is_same(Op, OpMul64) || V % 2 != 0) {
#pragma unroll
        for (int k = 0; k < V; ++k)
            w[k] = wave_incl64<Op>(e[k]);
    } else {
#pragma unroll
        for (int k = 0; k < V; k += 2) {
            uint64_t a = e[k], b = e[k + 1];
            if constexpr (__is_same(Op, OpAdd64)) {
                wave_incl64_add2(a, b);
            } else if constexpr (MaxFlip64<Op>::is) {
                constexpr uint64_t kFlip = MaxFlip64<Op>::mask;
                a ^= kFlip;
                b ^= kFlip;
                wave_incl64_max2(a, b);
                a ^= kFlip;
                b ^= kFlip;
            } else {
                wave_incl64_pair<Op>(a, b);
            }
            w[k] = a;
            w[k + 1] = b;
        }
    }
}

// Op with its operands swapped.
template <class Op>
struct Reversed64 {
    static constexpr uint64_t identity = Op::identity;
    __device__ static __forceinline__ uint64_t apply(uint64_t a, uint64_t b) { return Op::apply(b, a); }
};

__device__ __forceinline__ uint64_t wave_bcast_last64(uint64_t x)
{
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, 63);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(x >> 32), 63);
    return ((uint64_t)hi << 32) | lo;
}

template <class Op>
__device__ __forceinline__ uint64_t wave_fold64(uint64_t x)
{
    return wave_bcast_last64(wave_incl64<Op>(x));
}

// The previous lane's value (Op's identity in lane 0).
template <class Op>
__device__ __forceinline__ uint64_t wave_shr1_64(uint64_t x)
{
    return dpp64_or<kDppWaveShr1, 0xF>(x, Op::identity);
}

// Segmented inclusive wave scan of (head flag, value) pairs under
// (fa, va) . (fb, vb) = (fa | fb, fb ? vb : va + vb): a piece that holds a
// segment head does not take the sum from the pieces before it.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void seg_step(uint32_t &f, uint32_t &v)
{
    const uint32_t pf = dpp<CTRL, ROW_MASK>(f);
    const uint32_t pv = dpp<CTRL, ROW_MASK>(v);
    v = f ? v : v + pv;
    f |= pf;
}

__device__ __forceinline__ void wave_seg_incl(uint32_t &f, uint32_t &v)
{
    seg_step<kDppRowShr1, 0xF>(f, v);
    seg_step<kDppRowShr2, 0xF>(f, v);
    seg_step<kDppRowShr4, 0xF>(f, v);
    seg_step<kDppRowShr8, 0xF>(f, v);
    seg_step<kDppRowBcast15, 0xA>(f, v);
    seg_step<kDppRowBcast31, 0xC>(f, v);
}

// Zero, computed by an instruction that reads v: whatever uses the result is
// issued only after the load that wrote v has landed.
__device__ __forceinline__ int32_t zero_after(uint32_t v)
{
    uint32_t z;
    asm volatile("v_and_b32 %0, 0, %1" : "=v"(z) : "v"(v));
    return (int32_t)z;
}

// ---------------------------------------------------------------------------
// Chunk I/O.
// ---------------------------------------------------------------------------
__device__ __forceinline__ u32x4 load4(const uint32_t *abase, uint64_t q)
{
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(abase) + q);
}

__device__ __forceinline__ void store4(uint32_t *abase, uint64_t q, u32x4 v)
{
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(abase) + q);
}

// Chunk q with every element outside [vlo, vhi) read as 0.
__device__ __forceinline__ u32x4 load4_guarded(const uint32_t *abase, uint64_t q, uint64_t vlo,
                                               uint64_t vhi, uint32_t fill = 0u)
{
    u32x4 r = {fill, fill, fill, fill};
    const uint64_t v0 = q * 4;
    if (v0 >= vlo && v0 + 4 <= vhi)
        return load4(abase, q);
    if (v0 + 0 >= vlo && v0 + 0 < vhi) r.x = abase[v0 + 0];
    if (v0 + 1 >= vlo && v0 + 1 < vhi) r.y = abase[v0 + 1];
    if (v0 + 2 >= vlo && v0 + 2 < vhi) r.z = abase[v0 + 2];
    if (v0 + 3 >= vlo && v0 + 3 < vhi) r.w = abase[v0 + 3];
    return r;
}

// Store only the elements of chunk q inside [vlo, vhi).
__device__ __forceinline__ void store4_guarded(uint32_t *abase, uint64_t q, u32x4 v, uint64_t vlo,
                                               uint64_t vhi)
{
    const uint64_t v0 = q * 4;
    if (v0 >= vlo && v0 + 4 <= vhi) {
        store4(abase, q, v);
        return;
    }
    if (v0 + 0 >= vlo && v0 + 0 < vhi) abase[v0 + 0] = v.x;
    if (v0 + 1 >= vlo && v0 + 1 < vhi) abase[v0 + 1] = v.y;
    if (v0 + 2 >= vlo && v0 + 2 < vhi) abase[v0 + 2] = v.z;
    if (v0 + 3 >= vlo && v0 + 3 < vhi) abase[v0 + 3] = v.w;
}

// A tile's first chunk as a wave-uniform pointer (an SGPR pair): each lane
// then adds only a 32-bit offset, so all V loads or stores of a tile share
// one address register instead of holding V 64-bit addresses.
__device__ __forceinline__ u32x4 *uniform_tile_ptr(const uint32_t *abase, uint64_t vstart)
{
    const uint64_t q = vstart / 4;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)q);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(q >> 32));
    return const_cast<u32x4 *>(reinterpret_cast<const u32x4 *>(abase)) + (((uint64_t)hi << 32) | lo);
}

// A tile known to lie wholly inside the valid range.
template <int BLOCK, int V>
__device__ __forceinline__ void load_tile_full(const uint32_t *abase, uint64_t vstart,
                                               u32x4 (&x)[V])
{
    const u32x4 *t = uniform_tile_ptr(abase, vstart);
#pragma unroll
    for (int k = 0; k < V; ++k)
        x[k] = __builtin_nontemporal_load(t + (k * BLOCK + threadIdx.x));
}

template <int BLOCK, int V>
__device__ __forceinline__ void store_tile_full(uint32_t *abase, uint64_t vstart,
                                                const u32x4 (&x)[V])
{
    u32x4 *t = uniform_tile_ptr(abase, vstart);
#pragma unroll
    for (int k = 0; k < V; ++k)
        __builtin_nontemporal_store(x[k], t + (k * BLOCK + threadIdx.x));
}

// The loads of a whole tile at vstart, or -- when `real` is false -- the
// same number of loads of one 16-byte stand-in line.  The address is
// selected per load, so the instruction stream is the same either way: the
// compiler's count of outstanding loads then never depends on a branch.
template <int BLOCK, int V>
__device__ __forceinline__ void load_tile_full_or(const uint32_t *abase, uint64_t vstart,
                                                  const uint32_t *line, bool real,
                                                  u32x4 (&x)[V])
{
    const u32x4 *tile = uniform_tile_ptr(abase, vstart);
    const u32x4 *alt = reinterpret_cast<const u32x4 *>(line);
#pragma unroll
    for (int k = 0; k < V; ++k)
        x[k] = __builtin_nontemporal_load(real ? tile + (k * BLOCK + threadIdx.x) : alt);
}

// Any tile: whole tiles take the plain path, partial ones per-element guards.
template <int BLOCK, int V>
__device__ __forceinline__ void load_tile(const uint32_t *abase, uint64_t vstart, uint64_t vlo,
                                          uint64_t vhi, u32x4 (&x)[V], uint32_t fill = 0u)
{
    constexpr uint64_t T = (uint64_t)BLOCK * V * 4;
    if (vstart >= vlo && vstart + T <= vhi) {
        load_tile_full<BLOCK, V>(abase, vstart, x);
    } else {
        const uint64_t q0 = vstart / 4 + threadIdx.x;
#pragma unroll
        for (int k = 0; k < V; ++k)
            x[k] = load4_guarded(abase, q0 + (uint64_t)k * BLOCK, vlo, vhi, fill);
    }
}

template <int BLOCK, int V>
__device__ __forceinline__ void store_tile(uint32_t *abase, uint64_t vstart, uint64_t vlo,
                                           uint64_t vhi, const u32x4 (&x)[V])
{
    constexpr uint64_t T = (uint64_t)BLOCK * V * 4;
    if (vstart >= vlo && vstart + T <= vhi) {
        store_tile_full<BLOCK, V>(abase, vstart, x);
    } else {
        const uint64_t q0 = vstart / 4 + threadIdx.x;
#pragma unroll
        for (int k = 0; k < V; ++k)
            store4_guarded(abase, q0 + (uint64_t)k * BLOCK, x[k], vlo, vhi);
    }
}

// Stores that stream past the caches: non-temporal and device-scope, so a
// line leaves the L2 at once instead of waiting there dirty for an
// eviction.  For kernels that read no look-back descriptors: with
// device-scope descriptor reads in flight these stores were slower than
// plain non-temporal ones.
constexpr int kStreamStoreAux = 2 | 16;  // nt, sc1

// A whole tile's stores, device-scope and non-temporal, at virtual start vs
// of a 16-byte aligned base (vs a multiple of 4).
template <int BLOCK, int V>
__device__ __forceinline__ void store_tile_stream(uint32_t *abase, uint64_t vs,
                                                  const u32x4 (&x)[V])
{
    constexpr uint32_t kBytes = (uint32_t)BLOCK * V * 16;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(abase + vs, 0, kBytes, 0x00020000);
#pragma unroll
    for (int k = 0; k < V; ++k)
        __builtin_amdgcn_raw_buffer_store_b128(x[k], rs, (k * BLOCK + threadIdx.x) * 16, 0,
                                               kStreamStoreAux);
}

// u64 arrays use the same 16-byte chunks, two elements each: the virtual
// index is v = i + head with head = (address / 8) mod 2, so virtual chunk q
// holds u64 elements 2q and 2q + 1 (lanes x, y and z, w of the u32x4).
__device__ __forceinline__ uint64_t chunk_lo64(const u32x4 &c) { return ((uint64_t)c.y << 32) | c.x; }
__device__ __forceinline__ uint64_t chunk_hi64(const u32x4 &c) { return ((uint64_t)c.w << 32) | c.z; }
__device__ __forceinline__ u32x4 chunk_of64(uint64_t e0, uint64_t e1)
{
    return u32x4{(uint32_t)e0, (uint32_t)(e0 >> 32), (uint32_t)e1, (uint32_t)(e1 >> 32)};
}

// Chunk q of a u64 array with every element outside [vlo, vhi) read as fill.
__device__ __forceinline__ u32x4 load2_guarded64(const uint64_t *abase, uint64_t q, uint64_t vlo,
                                                 uint64_t vhi, uint64_t fill)
{
    const uint64_t v0 = q * 2;
    if (v0 >= vlo && v0 + 2 <= vhi)
        return load4(reinterpret_cast<const uint32_t *>(abase), q);
    const uint64_t e0 = (v0 >= vlo && v0 < vhi) ? abase[v0] : fill;
    const uint64_t e1 = (v0 + 1 >= vlo && v0 + 1 < vhi) ? abase[v0 + 1] : fill;
    return chunk_of64(e0, e1);
}

// Store only the u64 elements of chunk q inside [vlo, vhi).
__device__ __forceinline__ void store2_guarded64(uint64_t *abase, uint64_t q, u32x4 c,
                                                 uint64_t vlo, uint64_t vhi)
{
    const uint64_t v0 = q * 2;
    if (v0 >= vlo && v0 + 2 <= vhi) {
        store4(reinterpret_cast<uint32_t *>(abase), q, c);
        return;
    }
    if (v0 >= vlo && v0 < vhi) abase[v0] = chunk_lo64(c);
    if (v0 + 1 >= vlo && v0 + 1 < vhi) abase[v0 + 1] = chunk_hi64(c);
}

// ---------------------------------------------------------------------------
// Tile-local scan, in three phases around the caller's two barriers.
//
// Element order in a tile is (chunk k, thread, element), so the tile is V
// runs of BLOCK chunks.  Phase 1 scans each chunk in the thread and each
// run across the wave (DPP); lane 63 leaves the wave's total for run k in
// cell k*NW + wave of s_cell -- the cells in tile order.  After a barrier,
// phase 2 (one wave) turns the NW*V cells into their exclusive scan and
// returns the tile's sum.  After a second barrier, phase 3 adds to every
// element its cell's prefix, its lane's prefix inside the wave, and the
// carry from the tiles before.  Each thread reads only V cells, so the LDS
// values never crowd the registers that hold the tile.
// ---------------------------------------------------------------------------
template <int BLOCK, int V, class Op = OpAdd>
struct TileScan {
    static constexpr int NW = BLOCK / kWave;
    static constexpr int NCELL = NW * V;
    static constexpr int CELLS_PER_LANE = (NCELL + kWave - 1) / kWave;
    static constexpr bool kAdd = __is_same(Op, OpAdd);

    // Phase 1.  x[k] becomes the inclusive scan inside its chunk; w[k] the
    // inclusive wave scan of the chunk sums.
    __device__ static __forceinline__ void local(u32x4 (&x)[V], uint32_t (&w)[V],
                                                 uint32_t *s_cell)
    {
        const uint32_t wave = threadIdx.x / kWave;
#pragma unroll
        for (int k = 0; k < V; ++k) {
            x[k].y = Op::apply(x[k].y, x[k].x);
            x[k].z = Op::apply(x[k].z, x[k].y);
            x[k].w = Op::apply(x[k].w, x[k].z);
            w[k] = wave_incl<Op>(x[k].w);
        }
        if (lane_id() == kWave - 1) {
#pragma unroll
            for (int k = 0; k < V; ++k)
                s_cell[k * NW + wave] = w[k];
        }
    }

    // Phase 2, called by one whole wave after a barrier: the cells become
    // their exclusive scan; returns the tile's fold in every lane.
    __device__ static __forceinline__ uint32_t cells(uint32_t *s_cell)
    {
        // The mask tells the compiler lane < 64, so when the cells fill the
        // wave exactly the range checks fold away (no divergent reads).
        constexpr bool kExact = NCELL % kWave == 0;
        const uint32_t lane = lane_id() & (kWave - 1u);
        uint32_t v[CELLS_PER_LANE];
        uint32_t mine = Op::identity;
#pragma unroll
        for (int j = 0; j < CELLS_PER_LANE; ++j) {
            const uint32_t c = lane * CELLS_PER_LANE + j;
            v[j] = (kExact || c < (uint32_t)NCELL) ? s_cell[c] : Op::identity;
            mine = Op::apply(mine, v[j]);
        }
        const uint32_t incl = wave_incl<Op>(mine);
        uint32_t run;
        if constexpr (kAdd)
            run = incl - mine;
        else
            run = wave_shr1_op<Op>(incl);
#pragma unroll
        for (int j = 0; j < CELLS_PER_LANE; ++j) {
            const uint32_t c = lane * CELLS_PER_LANE + j;
            if (kExact || c < (uint32_t)NCELL)
                s_cell[c] = run;
            run = Op::apply(run, v[j]);
        }
        return wave_bcast_last(incl);
    }

    // Phase 3, after the barrier that follows phase 2: the tile's outputs
    // (exclusive or inclusive) combined with `carry`.
    template <bool INCL>
    __device__ static __forceinline__ void apply(u32x4 (&x)[V], const uint32_t (&w)[V],
                                                 const uint32_t *s_cell, uint32_t carry)
    {
        const uint32_t wave = threadIdx.x / kWave;
#pragma unroll
        for (int k = 0; k < V; ++k) {
            // Everything before this lane's chunk: the carry, the cells
            // before this (chunk, wave) run, the lanes before this one.
            uint32_t base;
            if constexpr (kAdd)
                base = carry + s_cell[k * NW + wave] + (w[k] - x[k].w);
            else
                base = Op::apply(Op::apply(carry, s_cell[k * NW + wave]), wave_shr1_op<Op>(w[k]));
            if (INCL) {
                x[k].x = Op::apply(base, x[k].x);
                x[k].y = Op::apply(base, x[k].y);
                x[k].z = Op::apply(base, x[k].z);
                x[k].w = Op::apply(base, x[k].w);
            } else {
                x[k].w = Op::apply(base, x[k].z);
                x[k].z = Op::apply(base, x[k].y);
                x[k].y = Op::apply(base, x[k].x);
                x[k].x = base;
            }
        }
    }
};

// ---------------------------------------------------------------------------
// Chained carry between tiles (decoupled look-back).
//
// Each launch draws tile numbers in arrival order from a 64-bit ticket word
// {high: epoch, low: next tile}.  A tile only waits on tiles with smaller
// numbers, which were drawn earlier by workgroups that are already running,
// so the wait always ends.  The tile that draws the last number resets the
// counter and advances the epoch, which readies the word for the next launch
// in stream order without any clearing.
//
// Each tile owns one 64-bit descriptor {high: epoch tag << 2 | status, low:
// value}, published with one agent-scope atomic store so value and status
// travel together.  A descriptor whose tag is not this launch's epoch is
// "not ready", so descriptors left by earlier launches are never believed.
//   status 1 (AGG):    value = this tile's own aggregate
//   status 2 (PREFIX): value = everything up to and including this tile
// ---------------------------------------------------------------------------
constexpr uint32_t kStatusAgg = 1;
constexpr uint32_t kStatusPrefix = 2;

struct TileTicket {
    uint32_t tile;
    uint32_t tag;   // (epoch mod 2^30) << 2
};

__device__ __forceinline__ TileTicket draw_ticket(uint64_t *ticket, uint32_t ntiles)
{
    const uint64_t old =
        __hip_atomic_fetch_add(ticket, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    TileTicket t;
    t.tile = (uint32_t)old;
    const uint32_t epoch = (uint32_t)(old >> 32);
    t.tag = (epoch & 0x3FFFFFFFu) << 2;
    if (t.tile == ntiles - 1)
        __hip_atomic_store(ticket, (uint64_t)(epoch + 1) << 32, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    return t;
}

__device__ __forceinline__ void publish(uint64_t *desc, uint32_t tile, uint32_t tag,
                                        uint32_t status, uint32_t value)
{
    const uint64_t word = ((uint64_t)(tag | status) << 32) | value;
    __hip_atomic_store(desc + tile, word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One look-back window: lane l holds the raw descriptor of tile base - l.
// Lanes before tile 0 read descriptor 0 and count as PREFIX 0.  The word is
// decoded only where it is used, so a caller can issue the load early and
// wait for it late.
struct LookbackWindow {
    uint64_t d;
    bool before_start;
};

// The lane number, computed afresh where it is used.  In a kernel at its
// register limit, a loop-invariant copy (or a 64-bit value derived from it)
// held across the tile loop is what the allocator spills first, and the
// reload then waits for every load and store the wave has in flight (the
// one-bit radix pass: +3.3%).
__device__ __forceinline__ uint32_t lane_id_here()
{
    uint32_t l = lane_id();
    asm volatile("" : "+v"(l));
    return l;
}

template <bool FRESH_LANE = false>
__device__ __forceinline__ LookbackWindow lookback_load(const uint64_t *desc, int64_t base)
{
    const int64_t pi = base - (int64_t)(FRESH_LANE ? lane_id_here() : lane_id());
    LookbackWindow w;
    w.before_start = pi < 0;
    w.d = __hip_atomic_load(desc + (pi < 0 ? 0 : pi), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return w;
}

// Folds one window into `excl` under Op.  Returns 2 when a PREFIX was
// reached (excl is the carry), 1 when all 64 tiles held aggregates (excl
// grew; look further back), 0 when a tile before the nearest PREFIX is not
// ready yet (nothing folded; read the same window again).  Lanes before tile
// 0 count as PREFIX with Op's identity.
template <class Op = OpAdd>
__device__ __forceinline__ int lookback_fold(const LookbackWindow &w, uint32_t tag,
                                             uint32_t &excl)
{
    const uint32_t hi = (uint32_t)(w.d >> 32);
    const uint32_t st = w.before_start ? kStatusPrefix : (((hi & ~3u) == tag) ? (hi & 3u) : 0u);
    const uint32_t val = w.before_start ? Op::identity : (uint32_t)w.d;
    const uint64_t pref = ballot(st == kStatusPrefix);
    const uint64_t wait = ballot(st == 0);
    const uint32_t p = pref ? (uint32_t)__builtin_ctzll(pref) : 64u;
    const uint64_t upto = (p >= 63) ? ~0ull : ((2ull << p) - 1);
    if (wait & upto)
        return 0;
    excl = Op::apply(excl, wave_fold<Op>(lane_id() <= p ? val : Op::identity));
    return pref ? 2 : 1;
}

// Called by one whole wave.  Returns, in every lane, the fold of the values
// of tiles tile-1, tile-2, ... back to and including the nearest PREFIX: the
// tile's exclusive carry.  Each step inspects 64 predecessors at once; `w` is
// the window for base = tile - 1, which a caller may have loaded early.  The
// first window is folded outside the retry loop, so waiting for it does not
// wait for loads the caller issued after it.
template <class Op = OpAdd, bool FRESH_LANE = false>
__device__ __forceinline__ uint32_t lookback_from(const uint64_t *desc, uint32_t tile,
                                                  uint32_t tag, LookbackWindow w)
{
    uint32_t excl = Op::identity;
    int r = lookback_fold<Op>(w, tag, excl);
    int64_t base = (int64_t)tile - 1;
    while (r != 2) {
        if (r == 1)
            base -= kWave;
        else
            __builtin_amdgcn_s_sleep(1);
        w = lookback_load<FRESH_LANE>(desc, base);
        r = lookback_fold<Op>(w, tag, excl);
    }
    return excl;
}

template <class Op = OpAdd>
__device__ __forceinline__ uint32_t lookback(const uint64_t *desc, uint32_t tile, uint32_t tag)
{
    return lookback_from<Op>(desc, tile, tag, lookback_load(desc, (int64_t)tile - 1));
}

// ---------------------------------------------------------------------------
// Chained carry of a u64 value: two descriptor words per tile, 2t holding
// {tag | status, low half} and 2t + 1 {tag | status, high half}.  Each word
// is one agent-scope atomic store, and a tile publishes each status once per
// launch, so a reader that finds the same tag and status in both words holds
// one publication's value; a pair caught between AGG and PREFIX disagrees
// and is read again, like a tile not yet ready.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void publish64(uint64_t *desc, uint32_t tile, uint32_t tag,
                                          uint32_t status, uint64_t value)
{
    const uint64_t head = (uint64_t)(tag | status) << 32;
    __hip_atomic_store(desc + 2 * (uint64_t)tile + 1, head | (value >> 32), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(desc + 2 * (uint64_t)tile, head | (uint32_t)value, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

struct LookbackWindow64 {
    uint64_t lo, hi;
    bool before_start;
};

__device__ __forceinline__ LookbackWindow64 lookback64_load(const uint64_t *desc, int64_t base)
{
    const int64_t pi = base - (int64_t)lane_id();
    const uint64_t q = pi < 0 ? 0 : (uint64_t)pi;
    LookbackWindow64 w;
    w.before_start = pi < 0;
    w.lo = __hip_atomic_load(desc + 2 * q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    w.hi = __hip_atomic_load(desc + 2 * q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return w;
}

// As lookback_fold, for u64 values, keeping operand order (tiles fold from
// the farthest to the nearest), so Op need not commute.
template <class Op>
__device__ __forceinline__ int lookback64_fold(const LookbackWindow64 &w, uint32_t tag,
                                               uint64_t &excl)
{
    const uint32_t hl = (uint32_t)(w.lo >> 32);
    const uint32_t hh = (uint32_t)(w.hi >> 32);
    const uint32_t st = w.before_start ? kStatusPrefix
                                       : (((hl & ~3u) == tag && hl == hh) ? (hl & 3u) : 0u);
    const uint64_t val =
        w.before_start ? Op::identity : (((uint64_t)(uint32_t)w.hi << 32) | (uint32_t)w.lo);
    const uint64_t pref = ballot(st == kStatusPrefix);
    const uint64_t wait = ballot(st == 0);
    const uint32_t p = pref ? (uint32_t)__builtin_ctzll(pref) : 64u;
    const uint64_t upto = (p >= 63) ? ~0ull : ((2ull << p) - 1);
    if (wait & upto)
        return 0;
    // Lane l holds tile base - l: the window's fold, farthest tile first, is
    // the lanes folded in descending order, and it goes before the nearer
    // windows already in excl.
    const uint64_t win = wave_fold64<Reversed64<Op>>(lane_id() <= p ? val : Op::identity);
    excl = Op::apply(win, excl);
    return pref ? 2 : 1;
}

template <class Op>
__device__ __forceinline__ uint64_t lookback64_from(const uint64_t *desc, uint32_t tile,
                                                    uint32_t tag, LookbackWindow64 w)
{
    uint64_t excl = Op::identity;
    int r = lookback64_fold<Op>(w, tag, excl);
    int64_t base = (int64_t)tile - 1;
    while (r != 2) {
        if (r == 1)
            base -= kWave;
        else
            __builtin_amdgcn_s_sleep(1);
        w = lookback64_load(desc, base);
        r = lookback64_fold<Op>(w, tag, excl);
    }
    return excl;
}

}  // namespace libscan
