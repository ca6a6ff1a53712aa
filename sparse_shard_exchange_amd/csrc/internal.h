// Internal host/device declarations of the pw library (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pw {

// Device status codes latched in the plan's status word (first error wins).
enum : uint32_t { ST_OK = 0, ST_BAD_DEST = 1, ST_TIMEOUT = 2 };

// Future-table rows. The table is [kNodes][width] of u32 epochs, a parallel
// [kNodes][width] of u32 fire counts and, when tracing, of u64 stamps.
enum : uint32_t { NODE_ARG = 0, NODE_A = 1, NODE_EXCH = 2, NODE_B = 3, NODE_RESULT = 4, NODE_STAGE = 5 };
constexpr uint32_t kNodes = 6;

enum : uint32_t { OP_IDENTITY = 0, OP_AFFINE = 1, OP_ROWSUM = 2 };

struct Futures {
  uint64_t* status;     // 1 word: the first error latched, code | (epoch of the call that latched it) << 32
  uint32_t* epoch;      // [kNodes][width]
  uint32_t* fires;      // [kNodes][width]
  uint64_t* stamps;     // [kNodes][width] or nullptr
  uint32_t width;
  uint32_t spin_ticks;  // bound of a device wait, in wall-clock ticks (100 MHz)
  uint32_t call_epoch;  // first epoch of the launching call (tags a latched error)
};

// Arguments of the exchange kernels (passed by value).
struct ExchangeArgs {
  const unsigned char* src;   // payload rows
  const int32_t* dest;        // [G]
  unsigned char* dst;         // [G] rows, exchange order
  int32_t* src_index;         // [G] or null
  int32_t* slot_of;           // [G] inverse of src_index (-1: dropped by the capacity) or null
  int32_t* counts;            // [num_src][N] or null
  int64_t* offsets_out;       // [N+1] or null
  void* b_out;                // B output or null
  uint64_t G;                 // tuples
  uint64_t dst_rows;          // rows dst can hold, at most G (slots past it are never written)
  uint32_t capacity;          // tuples kept per destination, first in tuple order (0 = all)
  uint64_t T;                 // tuples per source shard
  uint32_t N;                 // destinations
  uint32_t num_src;
  uint32_t row_bytes;         // payload bytes per tuple
  uint32_t fanout;            // payload row of tuple g is g / fanout
  uint32_t tile;              // tuples per workgroup tile (multiple of 256)
  uint32_t num_tiles;
  uint32_t scan_tiles, num_blk;  // tiles per scan block; scan blocks
  uint32_t fuse_scan;            // 1: the rank kernel also runs the scan (small tables)
  uint32_t nbits;             // bits needed to tell destinations apart
  uint32_t is_f32;
  uint32_t a_kind; float a_a, a_b;
  uint32_t b_kind; float b_a, b_b;
  uint32_t epoch;
  uint32_t b_gated;           // 1 if a B kernel follows and fires B futures itself
  Futures f;
  uint32_t* arrived;          // [N]
  uint32_t* expected;         // [N]
  uint32_t* b_arrived;        // [N]
  uint32_t* ctl;              // [0] result count, [1] scan done count
  uint32_t* tile_base;        // [num_tiles][N]: counts, then run starts inside the scan block
  uint32_t* blk_base;         // [num_blk][N]: block totals, then run starts inside the segment
  uint32_t* tile_cnt;         // [num_tiles][N]: counts (kept for the arrival counters)
  uint32_t* tile_done;        // [num_tiles]: scatter chunks finished
  uint16_t* rank;             // [G]: rank of tuple g among its tile's tuples with the same destination
  uint32_t chunk;             // tuples per scatter workgroup (a power of two dividing the tile)
  int64_t* seg;               // [N+1]
  // one-launch path (exchange_small.hip)
  uint32_t slab;              // tuples per workgroup (0: path not available)
  uint32_t call;              // one-launch calls of the plan so far, this one included
  uint64_t* slab_cnt;         // [grid][N] tuples per (slab, destination) | call << 32
  uint32_t* small_tab;        // [2][2N + 1]: arrivals, B arrivals, finished destinations, by call parity
};

// Arguments of the chain kernels (chain.hip).
struct ChainArgs {
  float* state;      // [N][E]: Arg of step 1, Result of the last step
  float* abuf;       // [N][E]: A's output
  uint32_t N, E;
  float a_a, a_b, b_a, b_b;
  uint32_t a_kind, b_kind;
  uint32_t epoch0;   // epoch (step) before this call
  uint32_t steps;
  uint32_t node;     // OpByOp: NODE_A or NODE_B
  uint32_t done_target;  // Result fires when the done counter reaches it
  uint32_t* done_ctr;
  uint32_t* role_ctr;    // split placement: [2] shards claimed for A, for B (cleared before each call)
  uint32_t* place;       // split placement: [N][2] XCD of the wave that ran A[i], B[i]
  uint32_t nxcc;         // XCDs of the device
  Futures f;
};

// Arguments of the persistent pipeline kernel (pipeline.hip).
struct PipeArgs {
  const __bf16* x;        // [M][rows][d] microbatch inputs
  __bf16* acts;           // [S][M][rows][d] stage outputs
  const __bf16* wt;       // [S][d][d] packed W_s^T ([out][in], K-contiguous)
  const uint32_t* order;  // [S M RB CT] tiles by queue, s | m << 8 | r << 16 | c << 24
  const uint32_t* qstart; // [nq] first order index of each queue
  const uint32_t* qlen;   // [nq] tiles in each queue
  uint32_t* qctr;         // [nq] claim counters (cleared before each pass)
  uint32_t nq;
  uint32_t* rb_ctr;       // [S][M][RB] column tiles finished per row block (cumulative)
  uint32_t* item_ctr;     // [S][M] row blocks finished (cumulative)
  uint32_t* done_ctr;     // workgroups finished (cumulative)
  uint32_t rb_target, item_target, done_target;
  uint32_t S, M, rows, d, RB, CT;
  uint32_t epoch;
  Futures f;
};

// Arguments of the mixture-of-experts kernels (moe.hip).
struct MoeArgs {
  const __bf16* x;         // [tokens][d]
  const __bf16* w1t;       // [E][hidden][d] packed W1^T
  const __bf16* w2t;       // [E][d][hidden] packed W2^T
  const __bf16* wrt;       // [64][d] packed W_r^T, experts >= E zero
  __bf16* xd;              // [2 tokens][d] dispatched rows (exchange output)
  __bf16* h;               // [2 tokens][hidden] FFN hidden activations
  __bf16* y;               // [2 tokens][d] expert outputs
  __bf16* out;             // [tokens][d] combined output
  float* logits;           // [tokens][E] or null
  int32_t* experts;        // [tokens][2]
  float* gates;            // [tokens][2]
  int32_t* slot_of;        // [2 tokens] dispatched slot of tuple g, -1 if dropped
  uint64_t tokens;
  uint32_t d, hidden, E;
  uint32_t max_row_blocks;  // upper bound of the expert row blocks (grid sizing)
  const int64_t* seg;      // [E+1] expert segment offsets (from the exchange)
  uint32_t* rb_start;      // [E+1] row-block prefix
  uint32_t* b_done;        // [E] finished FFN2 tiles
  uint32_t* ctl;           // [2] combine done counter
  uint32_t epoch;
  Futures f;
};

// Launchers (exchange.hip).
hipError_t launch_rank(const ExchangeArgs& a, hipStream_t s);
hipError_t launch_scan(const ExchangeArgs& a, hipStream_t s);
hipError_t launch_src_counts(const ExchangeArgs& a, hipStream_t s);
hipError_t launch_scatter(const ExchangeArgs& a, hipStream_t s);
hipError_t launch_b(const ExchangeArgs& a, hipStream_t s);
// exchange_small.hip: the whole step in one co-resident launch
uint32_t exchange_small_slab(uint64_t G, uint32_t N, uint32_t row_bytes, uint32_t b_kind, bool f32);
hipError_t launch_exchange_small(const ExchangeArgs& a, hipStream_t s);
uint32_t exchange_small_resident(int device);  // workgroups of the one-launch kernel the device holds at once
uint32_t scatter_chunk(uint32_t tile, uint32_t row_bytes, uint32_t fanout);
// mode: 0 chained (one launch, all steps), 1 one node (OpByOp), 2 fused.
// mode 3: split placement (A and B of a shard on different workgroups).
hipError_t launch_chain(const ChainArgs& a, uint32_t mode, hipStream_t s);
bool chain_split_fits(int device, uint32_t N, uint32_t E);  // every wave of the split placement resident at once
hipError_t launch_pipeline(const PipeArgs& a, uint32_t grid, hipStream_t s);
hipError_t launch_router(const MoeArgs& a, hipStream_t s);
hipError_t launch_moe_prefix(const MoeArgs& a, hipStream_t s);
hipError_t launch_ffn(const MoeArgs& a, bool second, uint32_t cus, hipStream_t s);
hipError_t launch_combine(const MoeArgs& a, hipStream_t s);
hipError_t launch_pack_t(const __bf16* in, __bf16* out, uint32_t batch, uint32_t K, uint32_t N_in, uint32_t N_out,
                         hipStream_t s);

}  // namespace pw
