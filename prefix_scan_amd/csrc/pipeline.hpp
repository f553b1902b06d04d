// pipeline.hpp -- the grid-filling two-tile driver of the chained carry,
// shared by every single-pass kernel of the library on gfx950.
//
// A chained carry makes each tile wait for the slowest of the tiles before
// it, and under a saturated HBM the loads of neighbouring tiles land
// microseconds apart.  Here a grid that fills the GPU once draws tile
// numbers from the ticket, and each workgroup holds two tiles in registers.
// Per step it
//   1. issues the current tile's first look-back window, draws the number of
//      the tile after next, and issues the loads of the next tile;
//   2. reduces the next tile locally and publishes its descriptor;
//   3. only then folds the current tile's carry, publishes its prefix, and
//      finishes the current tile (outputs and stores).
// So a tile asks for its carry one full load latency after its own
// aggregate went out, and its predecessors had the same time to publish.
//
// An Op that loads and reduces a tile in one call (load_local, below) has
// the window read later: once the next tile's loads have landed, just
// before that tile is reduced.  Read as the step starts, the window shows
// the descriptors of a load latency earlier, when the tiles just before --
// held by other workgroups at the same point of their own steps -- had not
// published their prefixes yet, so the fold mostly needed a second, fresh
// window: a round trip on the critical path.  Read late, it mostly holds a
// prefix already.
//
// Tile numbers are drawn one at a time (but for each workgroup's first two,
// drawn together), so consecutive tiles go to different workgroups that run
// side by side.  (Drawing several consecutive numbers
// per atomic would relieve the one contended ticket word, but it hands runs
// of consecutive tiles to one workgroup, which then finishes them one after
// another while the next workgroup waits on the last of them: the chain
// becomes serial.)  The ticket's rate -- one atomic per tile on one address
// -- is what keeps tiles large.
//
// Progress: every tile a workgroup holds lies above its current tile, and
// every drawn tile publishes its descriptor in step 2, as the next tile,
// without waiting on anything; a tile waits only on smaller ones.  So the
// workgroup with the smallest current tile looks back only over finished
// tiles, and always advances.  A workgroup stops at its first number past
// the end and counts itself out on the exit counter; the last one out resets
// the ticket (counter 0, epoch + 1) and the exit counter for the next
// launch, so no launch clears anything.
//
// The per-operation part is a policy type `Op`:
//   static constexpr int BLOCK;            threads per workgroup
//   using Monoid;                          the operator of the carry (OpAdd ...)
//   using Carry;                           (optional) Carry64<M> for a u64 carry
//   struct Regs;                           one tile's per-thread registers
//   struct Cells;                          one tile's LDS between phases
//   void load(Regs &, uint32_t tile);      issue the tile's loads
//   void local(Regs &, Cells &, uint32_t tile);   phase 1 (all threads)
//   TileInfoT<T> summary(Cells &, uint32_t tile); phase 2 (wave 0 only)
//   void finish(Regs &, Cells &, uint32_t tile, T carry);
//                                          outputs + stores (all threads;
//                                          may hold barriers of its own)
//   void last(T carry, const TileInfoT<T> &);     thread 0, last tile only
// where T is the carry's value type (u32 unless the Op names Carry64).
// Optionally, in place of load + local for the tile after the current one:
//   template <class R>
//   void load_local(Regs &, Cells &, uint32_t tile, R &&ready);
//                                          issue the loads, call ready(v) with
//                                          v a register the last load writes
//                                          (0 where there is none), then
//                                          phase 1
#pragma once

#include "device_common.hpp"

#include <type_traits>

namespace libscan {

// What phase 2 learned about a tile.
template <class T>
struct TileInfoT {
    T value;            // published value: the tile's aggregate, or -- when
                        // `final` -- its inclusive prefix already
    bool final;         // the value needs no carry (publish PREFIX at once)
    bool need_carry;    // the tile's outputs depend on the tiles before it
};
using TileInfo = TileInfoT<uint32_t>;

// How a carry of the monoid M travels between tiles: a u32 value in one
// descriptor word per tile (M must commute: the look-back folds nearer tiles
// first), or a u64 value in two (operand order kept, any associative M).
template <class M, bool FRESH_LANE = false>
struct Carry32 {
    using T = uint32_t;
    using Window = LookbackWindow;
    static constexpr T identity = M::identity;
    __device__ static __forceinline__ T apply(T a, T b) { return M::apply(a, b); }
    __device__ static __forceinline__ void put(uint64_t *desc, uint32_t t, uint32_t tag,
                                               uint32_t status, T v)
    {
        publish(desc, t, tag, status, v);
    }
    __device__ static __forceinline__ Window load(const uint64_t *desc, int64_t base)
    {
        return lookback_load<FRESH_LANE>(desc, base);
    }
    __device__ static __forceinline__ T from(const uint64_t *desc, uint32_t tile, uint32_t tag,
                                             const Window &w)
    {
        return lookback_from<M, FRESH_LANE>(desc, tile, tag, w);
    }
    // An empty use of the window's registers: the wait for its load is
    // taken at this point of the program.
    __device__ static __forceinline__ void settle(const Window &w) { asm volatile("" ::"v"(w.d)); }
};

template <class M>
struct Carry64 {
    using T = uint64_t;
    using Window = LookbackWindow64;
    static constexpr T identity = M::identity;
    __device__ static __forceinline__ T apply(T a, T b) { return M::apply(a, b); }
    __device__ static __forceinline__ void put(uint64_t *desc, uint32_t t, uint32_t tag,
                                               uint32_t status, T v)
    {
        publish64(desc, t, tag, status, v);
    }
    __device__ static __forceinline__ Window load(const uint64_t *desc, int64_t base)
    {
        return lookback64_load(desc, base);
    }
    __device__ static __forceinline__ T from(const uint64_t *desc, uint32_t tile, uint32_t tag,
                                             const Window &w)
    {
        return lookback64_from<M>(desc, tile, tag, w);
    }
    __device__ static __forceinline__ void settle(const Window &w)
    {
        asm volatile("" ::"v"(w.lo), "v"(w.hi));
    }
};

// An Op names its carry with `using Carry = ...`; without one it is the u32
// carry of its Monoid.
template <class Op, class = void>
struct carry_of {
    using type = Carry32<typename Op::Monoid>;
};
template <class Op>
struct carry_of<Op, std::void_t<typename Op::Carry>> {
    using type = typename Op::Carry;
};

constexpr uint32_t kNoTile = 0xFFFFFFFFu;

// Whether Op loads and reduces a tile in one call, with a hook between.
template <class Op, class = void>
struct has_load_local : std::false_type {};
template <class Op>
struct has_load_local<Op, std::void_t<decltype(Op::kLoadLocal)>> : std::true_type {};

template <class Op>
__device__ __forceinline__ void pipelined_chain(Op &op, uint32_t ntiles, uint64_t *ticket,
                                                uint32_t *exits, uint64_t *desc)
{
    constexpr int BLOCK = Op::BLOCK;
    constexpr int kDrawer = BLOCK - kWave;       // lane 0 of the last wave
    using C = typename carry_of<Op>::type;
    using CT = typename C::T;
    using Info = TileInfoT<CT>;
    // Three cell buffers in rotation: a tile's cells are written two steps
    // after the buffer's previous tile was last read, with barriers between.
    __shared__ typename Op::Cells s_cells[3];
    __shared__ uint32_t s_cur, s_nxt, s_nn, s_tag;
    __shared__ CT s_carry;

    auto tile_of = [&](uint32_t raw) -> uint32_t { return raw < ntiles ? raw : kNoTile; };
    auto draw_num = [&]() -> uint32_t {
        return __hip_atomic_fetch_add(reinterpret_cast<uint32_t *>(ticket), 1u, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
    };
    uint32_t epoch = 0;
    auto check_out = [&]() {                    // kDrawer, after its last draw
        const uint32_t before =
            __hip_atomic_fetch_add(exits, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (before == gridDim.x - 1) {
            __hip_atomic_store(exits, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(ticket, (uint64_t)(epoch + 1) << 32, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
    };

    if (threadIdx.x == kDrawer) {
        // The first two tiles in one draw: every workgroup draws before its
        // first load, and draws on the one ticket word are served one at a
        // time (~14 ns each), so a second draw here would double the wait
        // of the last workgroup to start (512 workgroups: ~14 against ~7 us).
        const uint64_t o1 =
            __hip_atomic_fetch_add(ticket, 2ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        epoch = (uint32_t)(o1 >> 32);
        const uint32_t c = tile_of((uint32_t)o1);
        const uint32_t x = c != kNoTile ? tile_of((uint32_t)o1 + 1u) : kNoTile;
        s_cur = c;
        s_nxt = x;
        s_tag = (epoch & 0x3FFFFFFFu) << 2;
        if (x == kNoTile)
            check_out();
    }
    __syncthreads();
    uint32_t cur = s_cur, nxt = s_nxt;
    const uint32_t tag = s_tag;
    if (cur == kNoTile)
        return;

    // Wave 0: a reduced tile's descriptor (tile 0's aggregate is its prefix).
    auto publish_info = [&](uint32_t t, const Info &in) {
        if (threadIdx.x == 0)
            C::put(desc, t, tag, (t == 0 || in.final) ? kStatusPrefix : kStatusAgg, in.value);
    };

    typename Op::Regs ra, rb;
    Info info_cur{C::identity, true, false};   // wave 0 only
    int cb = 0;                                 // cell buffer of `cur`

    // Prologue: the first tile, loaded and reduced synchronously.
    op.load(ra, cur);
    op.local(ra, s_cells[cb], cur);
    __syncthreads();
    if (threadIdx.x < kWave) {
        info_cur = op.summary(s_cells[cb], cur);
        publish_info(cur, info_cur);
    }

    // One step: X holds `cur` (reduced, descriptor out), Y receives `nxt`.
    auto step = [&](typename Op::Regs &X, typename Op::Regs &Y) {
        const int nb = cb == 2 ? 0 : cb + 1;
        const bool carry_needed = cur != 0 && info_cur.need_carry;     // wave 0
        const bool have_next = nxt != kNoTile;
        constexpr bool kLate = has_load_local<Op>::value;
        typename C::Window w0{};
        if (!kLate && threadIdx.x < kWave && carry_needed)
            w0 = C::load(desc, (int64_t)cur - 1);
        const bool drawing = threadIdx.x == kDrawer && nxt != kNoTile;
        const uint32_t nn_raw = drawing ? draw_num() : 0u;
        if (have_next) {
            if constexpr (kLate) {
                // The window is read after the load that writes `landed`
                // (and so after every earlier load: loads land in order).
                op.load_local(Y, s_cells[nb], nxt, [&](uint32_t landed) {
                    if (threadIdx.x < kWave && carry_needed)
                        w0 = C::load(desc, (int64_t)cur - 1 + zero_after(landed));
                });
            } else {
                op.load(Y, nxt);
                op.local(Y, s_cells[nb], nxt);
            }
        } else if (kLate && threadIdx.x < kWave && carry_needed) {
            w0 = C::load(desc, (int64_t)cur - 1);
        }
        __syncthreads();
        // A late window is still in flight here; every wave takes it now,
        // before anything is published.  A wave's one vector-memory counter
        // covers stores as well as loads, and the compiler keeps a load that
        // one branch issues and another consumes outstanding until a full
        // wait.  Taken later, that wait fell after the descriptor stores, so
        // wave 0 -- and the barrier after it -- waited for their write
        // acknowledgements every step (the u32 scan of 2^28 in place:
        // 338.4 -> 333.6 us; u64 scans 3-4% faster).  Here it waits only for
        // the window, which the fold needs first anyway.  (An early window
        // has landed with the next tile's loads.)
        if constexpr (kLate)
            C::settle(w0);
        Info info_next{C::identity, true, false};
        if (threadIdx.x < kWave) {
            if (have_next) {
                info_next = op.summary(s_cells[nb], nxt);
                publish_info(nxt, info_next);
            }
            CT excl = C::identity;
            if (carry_needed)
                excl = C::from(desc, cur, tag, w0);
            if (threadIdx.x == 0) {
                if (cur != 0 && !info_cur.final)
                    C::put(desc, cur, tag, kStatusPrefix, C::apply(excl, info_cur.value));
                s_carry = excl;
                if (cur == ntiles - 1)
                    op.last(excl, info_cur);
            }
        }
        if (threadIdx.x == kDrawer) {
            const uint32_t nn = drawing ? tile_of(nn_raw) : kNoTile;
            s_nn = nn;
            if (drawing && nn == kNoTile)
                check_out();
        }
        __syncthreads();
        op.finish(X, s_cells[cb], cur, s_carry);
        const uint32_t nn = s_nn;
        cur = nxt;
        nxt = nn;
        info_cur = info_next;
        cb = nb;
    };

    // Two steps per trip so the register sets swap roles without copies.
    for (;;) {
        step(ra, rb);
        if (cur == kNoTile)
            break;
        step(rb, ra);
        if (cur == kNoTile)
            break;
    }
}

}  // namespace libscan
