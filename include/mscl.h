/*
 * mscl.h — C ABI of a MemoryChannel-style AllReduce over R emulated peer
 * ranks held in one AMD Instinct MI355X (gfx950).
 *
 * What is emulated.  The MSCCL++ pages build their communication on
 * "channels": one GPU's link to one peer, set up by host code, handed to the
 * GPU once at start-up, and driven from kernel code through device functions
 * put / get / signal / flush / wait (MSCCL++ README, Key Concepts, "On-GPU
 * Communication Interfaces: Channels").  A MemoryChannel moves data with GPU
 * threads reading and writing the peer's memory directly (same page,
 * "PortChannel and MemoryChannel").  The pages' collective library offers
 * AllReduce for tensor-parallel serving (MSCCL++ project summary,
 * "Highlighted Details"; MSCCL++ ASPLOS'26 abstract).  Here the R ranks are
 * R groups of workgroups of one kernel, each rank's "remote" memory is a
 * buffer in the same GPU's HBM, and the channel semaphores are counters in
 * global memory.
 *
 * Result.  Every output buffer receives the element-wise sum of all R input
 * buffers, accumulated in binary32 in rank order 0..R-1 starting from rank
 * 0's value, then rounded once to the element type with round-to-nearest-even
 * (subnormals kept, NaN/Inf propagated).  The pages fix no accumulation rule;
 * this is the reading taken, and it makes one-shot and two-shot results
 * bit-identical to each other.
 *
 * Threading and concurrency.  Calls on one channel set (one device, one R)
 * share its semaphores, so they must be ordered on one stream (or otherwise
 * serialised).  Every kernel that runs a barrier (mscl_plan_t.uses_barrier)
 * needs all of its workgroups resident at once, and each launch is sized to
 * fit an otherwise idle device.  Kernels without a barrier running at the
 * same time on other streams only delay such a launch.  Two barrier-running
 * calls on different channel sets may overlap on concurrent streams only if
 * their grids fit the device together; the held two-shot
 * (mscl_plan_t.held_tiles > 0) takes all of a compute unit's LDS, so it must
 * not overlap any other barrier-running call (order such calls with events,
 * or run them on one stream).  A call that breaks this does not hang: its
 * bounded waits expire, TIMEOUT is recorded, and its outputs are wrong.  The
 * registry itself is thread-safe.
 *
 * Errors.  Every entry point returns a status code and never aborts.  The
 * text of the last failure on the calling thread is available from
 * mscl_last_error_string().  Argument validation runs on the host before any
 * HIP call.
 */
#ifndef MSCL_H
#define MSCL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MSCL_MAX_RANKS 16
#define MSCL_VERSION_MAJOR 0
#define MSCL_VERSION_MINOR 1
#define MSCL_VERSION_PATCH 0

typedef enum {
  MSCL_FLOAT32 = 0,  /* IEEE binary32 */
  MSCL_FLOAT16 = 1,  /* IEEE binary16 */
  MSCL_BFLOAT16 = 2  /* bfloat16 (upper half of a binary32 pattern) */
} mscl_dtype_t;

typedef enum {
  MSCL_ALGO_AUTO = 0,          /* by size: one-shot, then fused two-shot, then two-shot */
  MSCL_ALGO_ONE_SHOT = 1,      /* every rank reads all R inputs and writes its own output */
  MSCL_ALGO_TWO_SHOT = 2,      /* reduce-scatter, device signal/wait barrier, all-gather put */
  MSCL_ALGO_TWO_SHOT_FUSED = 3, /* reduce-scatter whose all-gather puts go out from registers
                                   (no re-read of the reduced chunk), then the completion
                                   barrier: each rank signals its peers once its puts into
                                   their outputs are visible, and waits for theirs */
  MSCL_ALGO_TWO_SHOT_PORT = 4,  /* reduce-scatter in the kernel; the all-gather puts go through a
                                   port channel: each rank's last workgroup posts R-1 put
                                   requests to a host proxy thread, which copies them with the
                                   SDMA engines, and waits for their completion.  Never chosen
                                   by AUTO (see mscl_allreduce) */
  MSCL_ALGO_TWO_SHOT_FUSED_NOBARRIER = 5, /* MSCL_ALGO_TWO_SHOT_FUSED without the completion
                                   barrier: no signal or wait at all; completion is the end of
                                   the kernel on the stream, which covers every rank only
                                   because all ranks share one GPU.  A comparison variant,
                                   never chosen by AUTO */
  MSCL_ALGO_TWO_SHOT_PERTILE = 6 /* reduce-scatter into each rank's own output with a semaphore
                                   signal per finished tile, then an all-gather in which every
                                   rank gets each peer's reduced tiles from the peer's output,
                                   each tile as soon as its semaphore shows it finished (no
                                   barrier between the phases).  Never chosen by AUTO */
} mscl_algo_t;

typedef int mscl_status_t;
#define MSCL_SUCCESS 0
#define MSCL_ERR_INVALID_ARGUMENT 1 /* a null/overlapping pointer, bad R, dtype, algo or size */
#define MSCL_ERR_UNSUPPORTED 2      /* the device is not a gfx950 GPU */
#define MSCL_ERR_MISALIGNED 3       /* a buffer is misaligned (16 bytes for allreduce, the element size for reduce-scatter and allgather) */
#define MSCL_ERR_NOT_INITIALIZED 4  /* no channel set exists for (current device, R) */
#define MSCL_ERR_OUT_OF_MEMORY 5    /* channel state could not be allocated */
#define MSCL_ERR_HIP 6              /* a HIP runtime call or kernel launch failed */
#define MSCL_ERR_TIMEOUT 7          /* a device-side wait() ran out of time */
#define MSCL_ERR_PROTOCOL 8         /* with protocol checks on (mscl_channel_set_checks): a semaphore held a
                                       count that calls ordered on one stream cannot produce */

typedef struct mscl_channel_s* mscl_channel_t;

/* Launch geometry chosen for one call (for tests and tooling). */
typedef struct {
  mscl_algo_t algo;          /* resolved algorithm (never AUTO) */
  int nranks;                /* R */
  int workgroups_per_rank;   /* B: workgroups (channel slots) per emulated rank */
  int threads_per_workgroup; /* 256; 128 for a fused two-shot too small to give each workgroup a 256-lane tile */
  int vectors_per_thread;    /* 16-byte vectors each thread keeps in flight per rank buffer */
  int uses_barrier;          /* 1 when the kernel runs the signal/wait barrier */
  size_t chunk_elems;        /* two-shot: elements owned by each rank (a multiple of 16/elem_size) */
  int cached_puts;           /* two-shot kernels: 1 when the puts into the outputs are device-scope
                                temporal stores (the call's 2*R*S bytes fit the Infinity Cache well,
                                and the outputs stay there for their next reader: up to 128 MiB, or
                                256 MiB for the held two-shot), 0 when they stream past the caches.
                                MSCL_CACHED_PUTS_MAX_BYTES (environment, read once) replaces the
                                built-in bounds on 2*R*S */
  int held_tiles;            /* two-shot, R >= 6: reduced tiles per lane each workgroup keeps in LDS
                                across the barrier instead of storing and re-reading them (its whole
                                share, 4 to 40 tiles), 0 when none.  MSCL_TWO_SHOT_HOLD=0 (environment, read once)
                                turns it off, and the slicing below with it */
  int slices;                /* kernel launches the call runs as: 1, or, for a two-shot too large for its
                                shares to fit in LDS, consecutive slices of slice_elems elements (the
                                last one shorter), each a complete two-shot; the fields above then
                                describe the first slice */
  size_t slice_elems;        /* elements per slice (count when slices == 1) */
  int tile_interleave;       /* sliced held two-shot, R <= 8: 1 when each slice that is a whole number of R
                                tiles deals its tiles to the ranks in turn (tile T to rank T mod R) instead
                                of giving each rank one contiguous chunk (a ragged last slice keeps chunks).
                                MSCL_TILE_INTERLEAVE=0 (environment, read once) turns it off */
} mscl_plan_t;

/*
 * Library version as MAJOR*10000 + MINOR*100 + PATCH.  The pages are silent
 * on versioning; this is bookkeeping of this library.  Never fails.
 */
int mscl_version(void);

/*
 * Static text for a status code ("unknown status" for anything else).  The
 * pages are silent on error reporting; the codes are this library's (every
 * entry point returns one instead of aborting).  The string is owned by the
 * library and lives as long as the process.  Never fails.
 */
const char* mscl_status_string(mscl_status_t status);

/*
 * Text describing the most recent failure on the calling thread ("" if
 * none).  The pages are silent; this library's diagnostics.  The string is
 * owned by the library and valid until the thread's next failing call.
 */
const char* mscl_last_error_string(void);

/*
 * Create (or reference) the channel set for `nranks` emulated ranks on HIP
 * device `device`.
 *   nranks : 1..MSCL_MAX_RANKS.
 *   device : HIP device ordinal; must be a gfx950 GPU.
 *   out    : receives the handle (non-null).
 * The host builds the channel state once and the kernels receive it by value
 * at launch, as the pages' channels are made by host code and handed to the
 * GPU at start-up (MSCCL++ README, Key Concepts, Channels).  State
 * owned by the library: per (receiver rank, sender rank, slot) semaphore
 * counters and per (rank, slot) consumed-signal counters in device memory, a
 * status word in host-mapped memory, and the slot count derived from the
 * kernels' occupancy so that every workgroup taking part in a barrier is
 * resident at once.  A second create for the same (device, nranks) returns
 * the same handle with its reference count raised.  Leaves the current
 * device unchanged.
 * Errors: INVALID_ARGUMENT, UNSUPPORTED, OUT_OF_MEMORY, HIP.
 */
mscl_status_t mscl_channel_create(int nranks, int device, mscl_channel_t* out);

/*
 * Drop one reference; the state is freed when the count reaches zero (the
 * port channel's proxy thread, if one was started, is stopped and joined
 * first).  The pages describe channels built by host code at start-up
 * (MSCCL++ README, Key Concepts, "On-GPU Communication Interfaces:
 * Channels") and are silent on their teardown; this is the counterpart of
 * mscl_channel_create.  The caller must have synchronised every stream that
 * used the set; graphs captured with calls on it must not be replayed
 * afterwards.
 *   channel : a handle from mscl_channel_create (not yet fully released).
 * Errors: INVALID_ARGUMENT (null or unknown handle), HIP.
 */
mscl_status_t mscl_channel_destroy(mscl_channel_t channel);

/*
 * Report a failure recorded by an earlier call on this set: a wait() that
 * ran out of time (TIMEOUT), a semaphore count that ordered calls cannot
 * produce (PROTOCOL, with mscl_channel_set_checks), or a port-channel request the proxy refused
 * (INVALID_ARGUMENT: a range outside the device allocations) or could not
 * issue (HIP).  The pages' wait() blocks until the peer signals (MSCCL++
 * README, Key Concepts, "On-GPU Communication Interfaces: Channels") and are
 * silent on a peer that never does; bounding the wait and recording the
 * failure here is this library's reading.  Reads the host-mapped status
 * word; it does not synchronise, so synchronise the stream first for a
 * complete answer.  Returns SUCCESS or the recorded code (INVALID_ARGUMENT
 * also for a null or unknown handle).
 */
mscl_status_t mscl_channel_check(mscl_channel_t channel);

/*
 * Zero the semaphores, the consumed-signal counters and the status word
 * (synchronous; the device must be idle on this set).  Needed after a
 * TIMEOUT, whose missing signals leave the counters out of step.  The pages
 * are silent on recovery from a lost signal; this is the library's.  A port
 * channel keeps its allocations (graphs captured earlier still point at
 * them): its proxy is stopped, its ring and counters zeroed, and the proxy
 * started again.
 * Errors: INVALID_ARGUMENT, HIP.
 */
mscl_status_t mscl_channel_reset(mscl_channel_t channel);

/*
 * AllReduce (sum) over R emulated ranks: the collective MSCCL++ accelerates
 * for tensor-parallel LLM serving (MSCCL++ project summary, "Highlighted
 * Details"), built on MemoryChannel-style device methods (MSCCL++ README,
 * Key Concepts, "On-GPU Communication Interfaces: Channels": put, signal,
 * wait; "PortChannel and MemoryChannel": many GPU threads loading and
 * storing the peer's memory).  The name and parameter list are fixed by the
 * target specification, which the pages do not give.
 *   inputs  : host array of nranks device pointers; inputs[r] is rank r's
 *             buffer of `count` elements.  Read only.  Inputs may alias each
 *             other.
 *   outputs : host array of nranks device pointers; outputs[r] receives the
 *             reduced buffer (count elements).  outputs[r] may equal
 *             inputs[r] (in place); otherwise it must not overlap any input,
 *             and no two outputs may overlap.
 *   count   : elements per buffer; 0 is a no-op that launches nothing (as is
 *             nranks == 1 in place).
 *   dtype   : element type of inputs and outputs.
 *   nranks  : R, 1..MSCL_MAX_RANKS; a channel set for (current device, R)
 *             must exist (mscl_channel_create).
 *   algo    : MSCL_ALGO_AUTO, _ONE_SHOT, _TWO_SHOT, _TWO_SHOT_FUSED,
 *             _TWO_SHOT_PORT, _TWO_SHOT_FUSED_NOBARRIER or _TWO_SHOT_PERTILE.
 *             All give bit-identical results.
 *   stream  : hipStream_t on the current device (NULL = default stream).
 * Every pointer must be 16-byte aligned and on the current device.  The call
 * is asynchronous: it validates, launches one kernel on `stream` (one per
 * slice for a large two-shot, below) and returns.  The caller owns all buffers and keeps them alive until the stream
 * has finished.  Nothing is allocated or copied to the device per call: the
 * pointer tables travel in the kernel arguments.
 * A failure recorded by an earlier call (see mscl_channel_check) makes this
 * call return that code without launching, until mscl_channel_reset().
 * A two-shot whose per-workgroup shares are too large to keep in LDS runs
 * as consecutive slices of every buffer, each a complete two-shot on its own
 * element range, launched back to back on `stream` (mscl_channel_plan
 * reports the slices); the result is the same, as the sum is elementwise.
 * That held two-shot uses all of each compute unit's LDS, one workgroup per
 * compute unit: kernels on other streams that hold LDS delay its workgroups
 * until they finish, and another barrier-running call must not overlap it
 * (see Threading above); MSCL_TWO_SHOT_HOLD=0 (environment, read once)
 * avoids the kernel.
 * Cache policy of the two-shot kernels' puts: when the call's footprint
 * (R inputs + R outputs, 2*R*count*element size) is at most 128 MiB (256 MiB
 * for the two-shot that holds its reduced chunk in LDS) they are
 * device-scope temporal stores, which leave the outputs in the Infinity
 * Cache for the kernel that reads them next; above that they stream past
 * the caches (mscl_channel_plan reports the choice).  It
 * changes time only, never results.
 * MSCL_ALGO_TWO_SHOT_PERTILE uses the channels' get (read the peer's memory
 * directly) and a semaphore per tile instead of one barrier (MSCCL++
 * README, Key Concepts, "On-GPU Communication Interfaces: Channels": put,
 * get, signal, wait); it moves about (3R - 1) * S bytes, against 2R * S
 * for the held two-shot, so AUTO does not use it.
 * MSCL_ALGO_TWO_SHOT_PORT follows the pages' PortChannel (MSCCL++ README, Key
 * Concepts, "PortChannel and MemoryChannel", "Host-Side Communication
 * Proxy"): GPU threads only post requests, and a CPU proxy moves the data
 * with DMA engines.  The first such call on a channel set allocates the
 * request ring (host-mapped memory) and completion counters and starts the
 * proxy thread, once; later calls allocate nothing.  The kernel ends only
 * after the proxy has completed every put, so stream order still marks the
 * result as ready; if the proxy does not finish within the wait bound the
 * channel records TIMEOUT.  The proxy checks every request against the
 * device allocations before copying and records INVALID_ARGUMENT for one
 * that leaves them.  Each put costs the copy engines ~20 us of set-up, so
 * this algorithm is for moving data without compute units, not for speed.
 * Errors: INVALID_ARGUMENT, MISALIGNED, NOT_INITIALIZED, TIMEOUT, PROTOCOL, HIP.
 */
mscl_status_t mscl_allreduce(const void* const inputs[], void* const outputs[], size_t count,
                             mscl_dtype_t dtype, int nranks, mscl_algo_t algo, void* stream);

/*
 * mscl_allreduce for callers that cannot allocate memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation):
 * the same arguments, algorithms and results, but no channel set is needed
 * and nothing is allocated, neither at the first call nor later.  The
 * channel state (semaphores, consumed-signal counters, status word) lives in
 * a 128 KiB array in the library's device code, one per device, held until
 * the process ends; the first call on a device looks up that array's address
 * and the device's geometry (host queries only).  Every call clears the
 * words its barriers use (a fill kernel on `stream`, no memset) before it
 * launches them, so calls on one device must not overlap: two such calls
 * running at once on different streams race on the shared array.  Launch
 * geometry is the same as mscl_allreduce's except that the workgroups per
 * rank are capped so that the channel state fits the array.
 * MSCL_ALGO_TWO_SHOT_PORT is refused (INVALID_ARGUMENT): its proxy needs a
 * request ring.  A device-side wait that runs out of time is recorded only
 * in the array (nothing host-visible exists to report it), leaves that
 * call's outputs wrong, and does not affect later calls.
 * Errors: INVALID_ARGUMENT, MISALIGNED, UNSUPPORTED, HIP.
 */
mscl_status_t mscl_allreduce_noalloc(const void* const inputs[], void* const outputs[], size_t count,
                                     mscl_dtype_t dtype, int nranks, mscl_algo_t algo, void* stream);

/*
 * ReduceScatter (sum) over R emulated ranks — the two-shot's first half as a
 * standard collective (the pages' library offers the usual collective
 * interface: MSCCL++ ASPLOS'26 abstract).
 *   inputs    : host array of nranks device pointers; inputs[p] holds
 *               nranks * recvcount elements.  Read only; may alias each other.
 *   outputs   : host array of nranks device pointers; outputs[r] receives
 *               recvcount elements: element i is the sum over p of
 *               inputs[p][r * recvcount + i], accumulated in binary32 in rank
 *               order and rounded once (as mscl_allreduce).  outputs[r] may be
 *               block r of inputs[r] (in place); otherwise outputs must not
 *               overlap any input or each other.
 *   recvcount : elements per output block; 0 is a no-op.
 *   dtype, nranks, stream : as mscl_allreduce (a channel set for the current
 *               device and nranks must exist).
 * Pointers need element-size alignment.  When every block boundary is 16-byte
 * aligned the data moves as 16-byte vectors, otherwise element by element.
 * Each rank gets its block from every peer and writes only its own output, so
 * the call runs no barrier.  Asynchronous, one kernel, no allocation.
 * Errors: INVALID_ARGUMENT, MISALIGNED, NOT_INITIALIZED, TIMEOUT, PROTOCOL, HIP.
 */
mscl_status_t mscl_reduce_scatter(const void* const inputs[], void* const outputs[], size_t recvcount,
                                  mscl_dtype_t dtype, int nranks, void* stream);

/*
 * AllGather over R emulated ranks — the two-shot's second half as a standard
 * collective (the pages' library offers the usual collective interface:
 * MSCCL++ ASPLOS'26 abstract; the data moves by MemoryChannel puts: MSCCL++
 * README, Key Concepts, "On-GPU Communication Interfaces: Channels").
 *   inputs    : host array of nranks device pointers; inputs[r] holds
 *               sendcount elements.  Read only.
 *   outputs   : host array of nranks device pointers; outputs[p] receives
 *               nranks * sendcount elements: block r is a bit-for-bit copy of
 *               inputs[r].  inputs[r] may be block r of outputs[r] (in place,
 *               that block is then left as it is); otherwise inputs must not
 *               overlap any output, and outputs must not overlap each other.
 *   sendcount : elements per input block; 0 is a no-op.
 *   dtype, nranks, stream : as mscl_allreduce.
 * Each rank puts its block into every peer's output (a MemoryChannel put);
 * the call's completion on the stream is the completion point.
 * Pointers need element-size alignment (16-byte vectors when every block
 * boundary allows).  Asynchronous, one kernel, no allocation.
 * Errors: INVALID_ARGUMENT, MISALIGNED, NOT_INITIALIZED, TIMEOUT, PROTOCOL, HIP.
 */
mscl_status_t mscl_allgather(const void* const inputs[], void* const outputs[], size_t sendcount,
                             mscl_dtype_t dtype, int nranks, void* stream);

/*
 * The algorithm MSCL_ALGO_AUTO resolves to for an out-of-place call of this
 * size (bytes = count * element size).  The target specification asks for
 * one-shot and two-shot variants switched by message size; the pages are
 * silent on the switch point, so the bands are crossovers measured on
 * MI355X (every band's algorithm carries the method's synchronisation):
 *   one-shot        bytes <= 8 MiB (R <= 2), 2 MiB (R = 3), 1 MiB (R = 4
 *                   and 5), 512 KiB (R = 6 and 7), 256 KiB (R = 8..11),
 *                   128 KiB (R = 12..16);
 *   fused two-shot  (with its completion barrier) bytes <= 256 KiB
 *                   (R = 16), 1 MiB (R = 6, 7 and 9..15), 2 MiB (R = 8),
 *                   8 MiB (R = 5), 16 MiB (R = 4), every size (R = 2, 3);
 *   two-shot        above.
 * In-place calls (any outputs[r] == inputs[r]) skip the one-shot band: in
 * place the one-shot needs a barrier between loads and stores; in place the
 * fused band also reaches 8 MiB at R = 8 and every size at R = 5
 * (mscl_channel_plan reports the in-place choice).  Pure host
 * computation.  MSCL_ONESHOT_MAX_BYTES (environment, read once) replaces the
 * one-shot limit for every R.
 * Errors: INVALID_ARGUMENT.
 */
mscl_status_t mscl_select_algo(size_t count, mscl_dtype_t dtype, int nranks, mscl_algo_t* out);

/*
 * The launch geometry mscl_allreduce would use on this channel set for this
 * size and algorithm (in_place: 1 if any outputs[r] == inputs[r]).  The pages
 * are silent on launch geometry; this exposes the library's own planner to
 * tests and tools.  Pure host computation; writes *plan.
 * Errors: INVALID_ARGUMENT (null plan, unknown handle, dtype or algo, or a
 * size that overflows).
 */
mscl_status_t mscl_channel_plan(mscl_channel_t channel, size_t count, mscl_dtype_t dtype,
                                mscl_algo_t algo, int in_place, mscl_plan_t* plan);

/*
 * Failure-handling controls for tests (never needed in normal use).  The
 * pages are silent on failure handling; these let tests force the bounded
 * wait of this library's wait() (see mscl_channel_check) from the host.
 *   wait_timeout_us : bound on every device-side wait() of later calls on
 *                     this set, in microseconds, at most a day (0 restores
 *                     the default of MSCL_WAIT_TIMEOUT_MS or 2000 ms).
 *   drop_signal_rank: -1 for normal operation; r in 0..R-1 makes rank r skip
 *                     its signal() in later calls, so its peers' wait()s run
 *                     into the bound and record TIMEOUT.  Every kernel still
 *                     exits.
 * Errors: INVALID_ARGUMENT.
 */
mscl_status_t mscl_channel_set_fault_controls(mscl_channel_t channel, uint64_t wait_timeout_us,
                                              int drop_signal_rank);

/*
 * Protocol checks, a race detector for the concurrency contract above (the
 * pages are silent on it; the counters are this library's semaphores).
 *   check_protocol    : nonzero makes every device-side wait of later calls on
 *                       this set check the count it reads.  A barrier wait
 *                       for epoch e can only ever see e - 1, e or e + 1 from
 *                       calls ordered on one stream (the peer cannot signal
 *                       e + 1 before this slot signals e, nor this slot wait
 *                       for e before the peer reached e - 1); a per-tile wait
 *                       only counts between 0 and the tiles the peer signals
 *                       in the call.  Any other count (two calls overlapping
 *                       on one set, a reset while a call ran) is recorded as
 *                       MSCL_ERR_PROTOCOL in the status word, reported like
 *                       TIMEOUT, and the call carries on.  Costs a compare per
 *                       wait.  MSCL_CHECK_PROTOCOL=1 (environment, read once)
 *                       turns it on for every new channel set.
 *   double_signal_rank: test control, -1 for normal operation; r in 0..R-1
 *                       makes rank r signal every barrier and every tile
 *                       twice, as a second call on the same counters would,
 *                       so that the checks have something to find.  No wait
 *                       blocks longer than without it.
 * Both settings stay until changed; mscl_channel_reset clears the recorded
 * status and the counters, not these.
 * Errors: INVALID_ARGUMENT (unknown handle, double_signal_rank out of range).
 */
mscl_status_t mscl_channel_set_checks(mscl_channel_t channel, int check_protocol, int double_signal_rank);

/*
 * Check the channel contract on the device (for tests and bring-up; it
 * synchronises and allocates, unlike the collectives).  For `rounds` rounds,
 * every (rank, slot) workgroup writes a 4 KiB mailbox, signals and waits on
 * the publishing barrier, reads the mailbox of the next rank's same slot (a
 * workgroup on another XCD for R > 1) and compares it with what that peer
 * wrote before signalling, since the pages' signal promises that every write
 * issued before it has completed (MSCCL++ README, Key Concepts, Channels);
 * then a second, write-after-read barrier (the one the in-place one-shot
 * uses) must hold the peer back from overwriting its mailbox with the next
 * round's words until those reads are done; a word from the wrong round is
 * a mismatch too.
 *   mismatches : receives the number of 32-bit words read that differed
 *                (0 when the channel keeps its promise).
 * Errors: INVALID_ARGUMENT, TIMEOUT (a wait ran out of time), HIP.
 */
mscl_status_t mscl_channel_selftest(mscl_channel_t channel, uint32_t rounds, uint64_t* mismatches);

#ifdef __cplusplus
}
#endif

#endif /* MSCL_H */
