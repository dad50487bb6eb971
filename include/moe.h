/*
 * moe.h — C ABI of libmoe.so: one expert-parallel rank's share of an MoE layer
 * on one MI355X (gfx950), with the W token-owner ranks emulated as W
 * receive buffers in HBM.
 *
 * Source: the reading-notes page "MoE 计算-通信细粒度重叠：用 Tile 级信号把 All-to-All
 * 藏在 GEMM 背后" on Cui, Wingkvist and Ericsson, "Fine-grained Computation-
 * Communication Overlap via Tile-level Signaling and Scheduling for Mixture-of-
 * Experts" ("the tile-signal notes" below).  Section numbers are the notes'.
 *
 * Conventions for every entry point
 *   - Returns a moe_status (0 = MOE_OK).  Arguments are validated on the host
 *     before any HIP call; nothing is enqueued when validation fails.
 *   - Device pointers are plain device addresses (hipMalloc or a torch
 *     tensor's data_ptr()).  bf16 tensors are passed as uint16_t bit patterns
 *     and must be 16-byte aligned; int32/uint32/float tensors 4-byte aligned.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Every call is asynchronous on it; nothing synchronises with the host
 *     except moe_device_status.
 *   - The caller owns every buffer.  The library allocates no device memory
 *     (moe_expert_combine_noalloc's scratch is a static array of the code
 *     object), creates no streams or events, and keeps only a per-device
 *     cache of the compute-unit count, the LDS limit and that array's
 *     address.
 *   - Errors the device detects (an expert id out of range, a received-row
 *     count that disagrees with the routing, a consumer wait that timed out)
 *     are written to an error word inside the plan workspace and reported by
 *     moe_device_status.
 */
#ifndef MOE_EXPERT_TILE_MOE_H
#define MOE_EXPERT_TILE_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_EINVAL = 1,       /* bad shape, null or misaligned pointer, bad option */
  MOE_ECAPACITY = 2,    /* a size exceeds what the plan workspace was sized for */
  MOE_EHIP = 3,         /* a HIP runtime call failed */
  MOE_ETIMEOUT = 4,     /* device: the consumer's bounded wait for a tile flag ran out */
  MOE_EROUTING = 5,     /* device: expert id out of range, or R disagrees with the routing */
  MOE_EUNSUPPORTED = 6  /* no GPU, or a device other than gfx950 */
} moe_status;

/* The pages' statement of the problem (tile-signal notes §4.4, input of the
 * layout + schedule pseudo-code: routing, local rank, number of ranks, experts
 * per rank, tile height tb_M) plus the layer sizes and the segment merge
 * factor of §5.2. */
typedef struct moe_shape {
  int32_t world;            /* W: ranks, also the token owners; 1..64 */
  int32_t rank;             /* r: the rank whose share is computed; 0..W-1 */
  int32_t experts_per_rank; /* E_l; rank q hosts global experts [q*E_l, (q+1)*E_l); W*E_l <= 1024 */
  int32_t top_k;            /* k; 1..min(32, W*E_l) */
  int32_t hidden;           /* d; multiple of 256 */
  int32_t ffn;              /* f; multiple of 128 */
  int32_t tb_m;             /* row-band height tb_M; multiple of 32 in [32, 256] */
  int32_t mgb;              /* bands merged into one middle segment (§5.2); 1..64 */
  const int32_t* tokens;    /* HOST array [W]: tokens owned by each rank (T_o >= 0) */
  int64_t recv_rows;        /* R: rows of x_recv = (owner, token, slot) triples routed to rank r */
} moe_shape;

/* Sizes the caller allocates (moe_query_sizes). */
typedef struct moe_sizes {
  size_t plan_bytes;        /* device plan workspace (int32 arrays, 256-byte aligned pieces) */
  int64_t rows_cap;         /* rows to allocate for x_layout [rows_cap, d], h [rows_cap, f], y [rows_cap, d]:
                               R + E_l*(W-1)*(tb_M-1), the padding bound of §4.3 per local expert */
  int64_t bands_cap;        /* upper bound on row bands: floor(rows_cap / tb_M) + E_l*W */
  int64_t flags_count;      /* uint32 tile flags for moe_expert_combine: 2 * bands_cap * tiles per band */
  int64_t recv_rows_self;   /* T_r * k: rows of the rank's own receive buffer (input of moe_scale) */
} moe_sizes;

/* Byte offsets of the plan's arrays inside the workspace (all int32), for
 * inspection and tests.  Layout of the header (int32 words at hdr):
 *   [0] error (moe_status of the last device-detected error, 0 if none)
 *   [1] M  total layout rows          [2] B  bands        [3] remote bands
 *   [4] segments                      [5] remote segments
 *   [6] gate/up tiles                 [7] down tile flags used (2 * B * tiles per band)
 *   [8] consumer copy units           [9] received rows counted from the routing
 *   [10] gate/up row tiles            [11] down row tiles
 *   [12..13] uint64: 100 MHz wall clock when the last producer workgroup of
 *            the down GEMM ended (raised by every call, never reset)
 *   [14..15] uint64: the same for the last consumer workgroup
 *   [16] down row tiles holding remote rows (they precede the others)
 *   [18..19] copy-unit claims handed out and producers started in the
 *            overlapped down-GEMM launch (reset by the gate/up launch)
 *   [20] planner: raised by the plan builder once the group tables the pair
 *        placers need are in memory, cleared by the counting launch */
typedef struct moe_plan_view {
  size_t hdr;
  size_t c;          /* [E_l][W] rows of local expert e from owner o */
  size_t grp_off;    /* [E_l][W] start of group (e, o) inside X_e */
  size_t m_e;        /* [E_l] rows of X_e, padding included */
  size_t row_off;    /* [E_l + 1] start of X_e inside the layout */
  size_t rb;         /* [E_l] remote row bands of expert e */
  size_t order;      /* [E_l] experts in schedule order (rule (ii)) */
  size_t base;       /* [W][E_l] owner o's (token, slot) pairs with expert below r*E_l + e */
  size_t band_expert, band_dst, band_src_row, band_dst_off, band_valid;  /* [B], schedule order S */
  size_t seg_first, seg_nbands, seg_dst, seg_dst_off, seg_src_row, seg_rows, seg_unit; /* [segments] (+1 for seg_unit) */
  size_t src_index;  /* [rows_cap] received row of each layout row, -1 for padding (first M valid) */
  size_t pos;        /* [T_r][k] row of the rank's own receive buffer holding slot (t, j) */
  /* GEMM row tiles (implementation detail, for tests), as first compacted
   * row and expert per tile.  Gate/up: X_e's compacted rows cut into pieces
   * of 256, experts in rule (ii) order.  Down: the same pieces, those that
   * hold remote rows first (experts in rule (ii) order), then those of local
   * rows alone (experts ascending); a piece may end inside a band.
   * grp_band [E_l][W]: first band of group (e, o) in S. */
  size_t gu_tile_row, gu_tile_expert;   /* [hdr[10]] */
  size_t dn_tile_row, dn_tile_expert;   /* [hdr[11]] */
  size_t grp_band;
  /* uint64 [sk_counters_count]: epoch-tagged tile counters of the GEMMs'
   * K-split tails; zero them (with the flags) before an epoch is reused */
  size_t sk_counters, sk_counters_count;
  /* Compacted rows: the layout's R real rows without its padding, in layout
   * order (experts ascending, inside X_e the groups in layout order).  The
   * gate/up GEMM runs over them, so it computes no padding row, and h holds
   * them in this order.  crow_off [E_l + 1]: first compacted row of X_e;
   * grp_crow [E_l][W]: offset of group (e, o) inside X_e's compacted rows;
   * band_crow [B]: first compacted row of every band (schedule order);
   * cmp_row [R]: layout row of every compacted row; cmp_src [R]: its
   * received row (index into x_recv). */
  size_t crow_off, grp_crow, band_crow, cmp_row, cmp_src;
} moe_plan_view;

/* moe_expert_combine modes */
enum {
  MOE_MODE_OVERLAP = 0,   /* down GEMM and consumer run concurrently on disjoint CUs, one launch (§5.3) */
  MOE_MODE_SERIAL = 1,    /* down GEMM to completion, then the consumer on all CUs (serial baseline) */
  MOE_MODE_COPY_ONLY = 2, /* only the consumer, on the caller's stream; flags must already equal `epoch` */
  MOE_MODE_COPY_ROWS = 3  /* like COPY_ONLY, but the per-row ablation of the copy (tile-signal notes
                             §4.3, the alternative to the owner-aligned layout): each remote row is
                             routed and copied on its own, one wavefront per row, after its band's
                             flags; same result as the consumer, for measurement */
};

typedef struct moe_combine_opts {
  int32_t mode;             /* MOE_MODE_* */
  int32_t consumer_cus;     /* OVERLAP: CUs given to the consumer, multiple of 8 in [8, 128]; 0 = 16 */
  int32_t consumer_blocks;  /* workgroups of the consumer; 0 = consumer_cus (OVERLAP: at most
                               consumer_cus, MOE_EINVAL above) or one per 32 KiB copy unit,
                               bounded on the host (SERIAL, COPY_ONLY) */
  int32_t link_mbps;        /* 0: the consumer copies at memory speed.  > 0 (1000 at least): an
                               emulated link per destination rank in MB/s (an xGMI link is ~153000):
                               each copy unit to owner o also occupies owner o's link for
                               bytes / rate, reserved in order on the device clock, and the copying
                               workgroup waits until that transfer would have ended (COPY_ROWS
                               ignores it) */
  int64_t spin_timeout_ns;  /* bound on the consumer's wait for one segment's flags; 0 = 2 s */
  void* events[6];          /* optional hipEvent_t, recorded on `stream`: [0]/[1] around the gate/up GEMM,
                               [2]/[3] around the down GEMM, [4]/[5] around the consumer (in OVERLAP both
                               pairs bracket the one launch that runs both); NULL entries are skipped */
  const void* x_recv;       /* gathered rows: when x_layout is NULL, the gate/up GEMM reads layout row m
                               straight from x_recv[src_index[m]] (device bf16 [R, d], the array given to
                               moe_plan) and padding rows as zeros, so X is never materialized; requires
                               R*d*2 < 2^31 bytes; may be NULL when R = 0.  Ignored when x_layout is
                               given. */
  int32_t signal;           /* how the down GEMM tells the consumer that rows are ready:
                               MOE_SIGNAL_TILE (0): two flags per band and column tile (the band's
                               head and tail), set to `epoch` by the tile that computed them (the
                               consumer polls every flag of a segment); MOE_SIGNAL_GROUP (1): one
                               ready counter per (expert, destination) group, raised by every tile by
                               the band heads and tails of the group it holds and tagged with
                               `epoch` (the consumer polls one word per segment; a
                               segment waits for its whole group).  COPY_ONLY must use the mode
                               the compute call used; COPY_ROWS needs MOE_SIGNAL_TILE */
  int32_t pad;              /* zero */
} moe_combine_opts;

enum { MOE_SIGNAL_TILE = 0, MOE_SIGNAL_GROUP = 1 };

/* Text of a status code. */
const char* moe_status_string(int status);

/* Sizes the caller must allocate for `shape`. Host only; no HIP call. */
int moe_query_sizes(const moe_shape* shape, moe_sizes* out);

/* Offsets of the plan arrays inside the workspace. Host only; no HIP call. */
int moe_plan_offsets(const moe_shape* shape, moe_plan_view* out);

/*
 * moe_plan — Stage A of the tile-signal notes (§3, §4.2, §4.4, §4.5, §5.2):
 * builds, on the device, the owner-aligned row layout of every local expert
 * (rows grouped by owner; remote groups zero-padded to a multiple of tb_M,
 * ascending owner rank with r skipped; the local group last, unpadded), the
 * remote-first band schedule S (experts by remote band count, descending,
 * ties to the lower id; remote bands first), the combine plan (destination,
 * destination row, valid rows per band), the segments and the owner-side
 * slot table of rank r's own tokens, and writes the layout X.
 *   topk_ids  device int32 [N, k], N = sum(tokens): global expert ids of every
 *             owner's tokens, owner-major (owner 0's T_0 tokens first).  Only
 *             rows routed to rank r matter for X; owner r's rows give `pos`.
 *   x_recv    device bf16 [R, d]: the received rows in arrival order, i.e.
 *             every (owner, token, slot) with expert on rank r, lexicographic.
 *   plan_ws   device, plan_bytes from moe_query_sizes; written.
 *   x_layout  device bf16 [rows_cap, d]; rows [0, M) written (padding = +0).
 *             May be NULL: then only the metadata is built, X is not
 *             materialized, and moe_expert_combine must gather its rows from
 *             x_recv (moe_combine_opts.x_recv).
 * Owner o's receive buffer (see moe_expert_combine) is [T_o*k, d], ordered by
 * (global expert, token).  Errors in the routing are reported through the
 * error word; all later kernels of this plan then do nothing.
 */
int moe_plan(const moe_shape* shape, const int32_t* topk_ids, const uint16_t* x_recv,
             void* plan_ws, uint16_t* x_layout, void* stream);

/*
 * moe_expert_combine — Stage B of the tile-signal notes (§5): the SwiGLU
 * expert FFN of every local expert as grouped bf16 GEMMs over the layout, and
 * the combine.  The gate/up GEMM writes h = silu(X W_gate^T) * (X W_up^T)
 * (fp32 accumulation, h rounded once to bf16).  The down GEMM takes its tiles
 * in schedule order (workgroup i takes tiles i, i+g, ...; §5.1), writes
 * y = h W_down^T (bf16) and, in its epilogue, publishes the tile: its rows
 * are stored at device scope and acknowledged before the tile's flags are
 * set to epoch, so they are visible on every XCD first.  Each band has two
 * flags per column tile, one for its head and one for its tail, set by the
 * tile(s) holding them (a band may straddle two row tiles).  The consumer
 * waits (bounded) until every flag of a remote segment's bands is set, reads
 * the rows at device scope and copies the segment's valid rows to
 * recv[dst] + dst_off*d; padding rows are never copied.  Rows of local bands
 * (destination r) never leave the rank: the down GEMM's epilogue writes them
 * into recv[r] itself, besides y.
 *   x_layout   device bf16 [rows_cap, d] from moe_plan, or NULL with opts->x_recv set
 *              (gathered rows, see moe_combine_opts).
 *   w_gate_up  device bf16 [E_l, 2f, d]: rows 0..f-1 gate, f..2f-1 up (K-contiguous).
 *   w_down     device bf16 [E_l, d, f] (K-contiguous).
 *   h, y       device bf16 [rows_cap, f] and [rows_cap, d]; scratch written here:
 *              h holds the R real rows in compacted order (moe_plan_view), y
 *              every layout row of [0, M), zeros in the padding rows of
 *              remote bands; padding rows are never multiplied.
 *   flags      device uint32 [flags_count]; zero them once at allocation, then
 *              pass a new epoch (never 0, increasing) on every call: no reset.
 *              An epoch value may be used again only after the flags and the
 *              plan's sk_counters (moe_plan_view) are zeroed, e.g. when the
 *              32-bit epoch wraps around.
 *   recv       HOST array of W device pointers; recv[o] is bf16 [T_o*k, d].
 *   opts       may be NULL (OVERLAP, defaults).
 * Every mode runs on `stream` alone.  OVERLAP launches the down GEMM with
 * consumer_blocks extra workgroups past its producers; they take the last
 * CUs to be filled and copy while the producers compute.  Copy units are
 * claimed in schedule order from a counter in the plan header; producers
 * that run out of tiles claim units too, once every producer has started.
 * The plan header's claim counters are reset by the gate/up launch of the
 * same call, so two calls on one plan workspace must not overlap.
 */
int moe_expert_combine(const moe_shape* shape, const void* plan_ws, const uint16_t* x_layout,
                       const uint16_t* w_gate_up, const uint16_t* w_down,
                       uint16_t* h, uint16_t* y, uint32_t* flags, uint32_t epoch,
                       uint16_t* const* recv, const moe_combine_opts* opts, void* stream);

/*
 * moe_expert_combine_noalloc — moe_expert_combine for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, modes, results and
 * errors as moe_expert_combine, and it allocates nothing: the scratch of its
 * kernels (the fp32 partial sums of the GEMMs' K-split tails, their tile
 * counters, the copy-claim counters of the overlapped launch) is a static
 * device array of 64 MiB + 13 KiB that every GPU the library runs on holds
 * until the process ends; its device address is looked up once per device.
 * So the plan workspace only needs the first moe_plan_view.sk_counters
 * bytes of plan_bytes (the K-split part at its end is not used).
 * Limit: at most 256 partial-sum slots of 256 KiB.  No input is refused
 * for it: a K-split tail that would need more pieces than the slots allow
 * is cut into fewer, longer pieces, or not split at all, which changes only
 * the fp32 summation order of those tiles.
 * The counters are cleared at the start of every call (a small fill kernel
 * on `stream`).  Every call on one GPU shares that GPU's array: calls that
 * overlap on the device (other streams, or concurrent host threads) race and
 * give wrong results; calls on one stream never overlap.
 */
int moe_expert_combine_noalloc(const moe_shape* shape, const void* plan_ws, const uint16_t* x_layout,
                               const uint16_t* w_gate_up, const uint16_t* w_down,
                               uint16_t* h, uint16_t* y, uint32_t* flags, uint32_t epoch,
                               uint16_t* const* recv, const moe_combine_opts* opts, void* stream);

/*
 * moe_scale — step 5 of the distributed MoE forward (tile-signal notes §2.2;
 * §2.1: the output is the gate-weighted sum of the selected experts' outputs):
 *   out[t] = bf16( sum_{j<k} topk_w[t][j] * recv_self[pos[t][j]] ), fp32 in j order.
 *   recv_self  device bf16 [T_r*k, d]: rank r's own receive buffer.
 *   topk_w     device float [T_r, k]: gate weights of rank r's tokens.
 *   out        device bf16 [T_r, d].
 */
int moe_scale(const moe_shape* shape, const void* plan_ws, const uint16_t* recv_self,
              const float* topk_w, uint16_t* out, void* stream);

/* Synchronises `stream`, then returns the device error word of the plan
 * (MOE_OK, MOE_ETIMEOUT or MOE_EROUTING), or MOE_EHIP. */
int moe_device_status(const void* plan_ws, void* stream);

/* Number of compute units of the current device (0 without a GPU). */
int moe_device_cus(void);


#ifdef __cplusplus
}
#endif

#endif /* MOE_EXPERT_TILE_MOE_H */
