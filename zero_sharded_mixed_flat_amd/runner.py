"""One rank's ZeRO step over a workload, as a sequence of C-ABI calls.

``RankStep`` allocates the device buffers a workload needs (caller-owned, as
the ABI requires), fills them from the seeded generators, and runs steps:

    reduce each emulated owner's slice            zero_reduce_shard, or
                                                  zero_reduce_owners (all owners, one launch)  (a1)
    norm + clip multiplier over all owners        zero_grad_norm      (a2)
    AdamW + 16-bit cast into the parameter buffer zero_adam_step_owners (a3)
    per-unit gather of every rank's 16-bit shard  zero_gather_params  (a4)
    close the step: advance t if it was applied,
    clear the flag                                zero_step_end

With a block-quantised gather (ZeRO++ quantised weights) the last step is

    quantise the rank's updated 16-bit shard      zero_quantize_blocks
    per-unit gather of every rank's codes,
    dequantised into the 16-bit full buffer       zero_gather_dequant

With ZeRO-Offload the fp32 state is in host memory and the AdamW step is

    gradient to the host, host AdamW, 16-bit
    parameters back, chunk by chunk               zero_offload_adam_step

or, with the one-step-delayed update, the same chunked update started on a
thread of the library's while the GPU goes on with the next step, its
parameters applied when that step reaches its update

    the previous update's parameters in place     zero_offload_end
    gradient copied aside, host update started    zero_offload_begin

All calls go to one stream with no host synchronisation inside a step
(except the offloaded update, which waits for its copies): the clip
multiplier, the skip flag and the step count stay in device memory.  AdamW
takes its scalars from a device table of one zero_adam_consts per step,
indexed by the device step count, which only applied steps advance; so a
step skipped for a non-finite gradient leaves the bias corrections of the
next one unchanged, and a captured step replays with no host work at all.
Contributions of the emulated ranks are buffers in this GPU's memory (one
process, one GPU).
"""

import ctypes
import os

import torch

from . import abi, synth

OFFLOAD_CHUNK = 1 << 23          # values per staging slot of the offloaded update
CONSTS_TABLE_LEN = 1024          # steps of AdamW scalars held on the device at a time
CONTRIB_ROW_ALIGN = 2048         # 16-bit elements: 4 KiB
HOST_THREADS_MAX = 16

TORCH16 = synth.TORCH_DTYPES


class RankStep:
    def __init__(self, w, seed=0, device="cuda", tile_period=None):
        self.w = w
        self.seed = seed
        self.device = device
        self.plan = abi.Plan(w.units, w.nd, w.stage, w.align)
        self.n, _ = self.plan.rank(0)
        self.full_numel = self.plan.full_numel()
        info = self.plan.info()
        self.n_units = info["n_units"]
        self.owners = list(range(w.nd)) if w.all_ranks else [w.rank]
        gdt, pdt = TORCH16[w.grad_dtype], TORCH16[w.param_dtype]
        n = self.n
        dev = device

        self.ledger = []          # (buffer, role, bytes) of every allocation, in order

        # Gradients.  With every rank emulated on one flat unit, each rank holds a
        # full local gradient and owner o's contribution from rank r is the slice
        # [o*n, (o+1)*n) of rank r's gradient.  Otherwise this rank's own gradient
        # is the whole local gradient under ZeRO-0/1 (gradients are not sharded)
        # or only its slice under ZeRO-2/3, and the other ranks' contributions to
        # the slice are an [nd - 1, n] block standing in for their buffers.  The
        # reduce writes the average in place over the rank's own contribution,
        # where a rank keeps its reduced slice.
        self.local = None
        self.contrib_block = None
        self.grad_full = None
        self.own_grad = None
        row = -(-n // CONTRIB_ROW_ALIGN) * CONTRIB_ROW_ALIGN
        if w.pre_reduced:
            self.grad = self._keep("grad", "grads16",
                                   synth.grad16(n, w.grad_dtype, w.grad_std * w.loss_scale, seed, 1, dev))
            if tile_period:
                synth.tile_(self.grad, tile_period)
        elif w.all_ranks and self.n_units == 1:
            self.local = self._keep("local", "all_ranks_grads16",
                                    torch.empty((w.nd, self.full_numel), dtype=gdt, device=dev))
            self.fresh_gradients(step=0, tile_period=tile_period)
            self.reduced = self._keep("reduced", "all_ranks_grads16",
                                      torch.empty((len(self.owners), n), dtype=gdt, device=dev))
        else:
            # Rows start on 4 KiB boundaries, as separate (peer) buffers would:
            # a row stride of 2n bytes alone can leave every wave-wide access
            # straddling one more 128-byte line than it needs.
            if w.nd > 1:
                self.contrib_block = self._keep("peer_contributions", "peers",
                                                torch.empty((w.nd - 1, row), dtype=gdt, device=dev))[:, :n]
            if w.stage <= 1:
                self.grad_full = self._keep("grad_full", "grads16",
                                            torch.zeros(self.full_numel, dtype=gdt, device=dev))
                self.own_grad = self.grad_full[w.rank * n:(w.rank + 1) * n]
            else:
                self.own_grad = self._keep("grad_own", "grads16", torch.empty(row, dtype=gdt, device=dev))[:n]
            for r, c in enumerate(self.contribs(0)):
                synth.normal_(c, w.grad_std * w.loss_scale, seed, 100 + r)
                synth.outliers_(c, w.outlier_frac, w.outlier_mult, seed, 100 + r)
                if tile_period:
                    synth.tile_(c, tile_period)
            self.reduced = self.own_grad.view(1, n)

        # fp32 optimizer state, one shard per emulated owner (in host memory,
        # drawn on the GPU chunk by chunk, under ZeRO-Offload).
        k = len(self.owners)
        state_dev = "cpu" if w.offload else dev
        role = ("all_ranks_" if k > 1 else "") + ("state32_host" if w.offload else "state32")
        self.master = self._keep("master", role, torch.empty((k, n), dtype=torch.float32, device=state_dev))
        self.m = self._keep("m", role, torch.empty((k, n), dtype=torch.float32, device=state_dev))
        self.v = self._keep("v", role, torch.empty((k, n), dtype=torch.float32, device=state_dev))
        for i, o in enumerate(self.owners):
            synth.normal_(self.master[i], w.master_std, seed, 200 + o, via=dev)
            if w.m_std:
                synth.normal_(self.m[i], w.m_std, seed, 300 + o, via=dev)
            else:
                self.m[i].zero_()
            if w.v_std:
                synth.abs_normal_(self.v[i], w.v_std, seed, 400 + o, via=dev)
            else:
                self.v[i].zero_()
            if w.all_ranks:
                self._zero_padding(o, self.master[i])

        # 16-bit parameters.  ZeRO-1/2 write the owner's slice straight into the
        # full gather buffer; ZeRO-3 writes the owner's shard, then gathers every
        # rank's shard unit by unit into the full buffer (assembled layer by
        # layer for compute); a pre-reduced owner update writes its shard.
        self.full = None
        self.shards = None
        if w.gather_per_unit:
            if k > 1:
                block = self._keep("shards", "all_ranks_params16", torch.empty((w.nd, n), dtype=pdt, device=dev))
                self.shards = list(block)
                self._shards_block = block
            else:
                own = self._keep("shard_own", "params16", torch.empty(n, dtype=pdt, device=dev))
                peers = self._keep("peer_shards", "peers", torch.empty((w.nd - 1, n), dtype=pdt, device=dev))
                self.shards = [peers[r if r < w.rank else r - 1] for r in range(w.nd) if r != w.rank]
                self.shards.insert(w.rank, own)
            for r in range(w.nd):
                if r not in self.owners:
                    synth.normal_(self.shards[r], w.gather_shard_std, seed, 500 + r)
            self.full = self._keep("gathered", "gathered", torch.zeros(self.full_numel, dtype=pdt, device=dev))
        elif w.pre_reduced:
            self.param = self._keep("param", "params16", torch.zeros(n, dtype=pdt, device=dev))
        else:
            self.full = self._keep("full", "all_ranks_params16" if k > 1 else "params16",
                                   torch.zeros(self.full_numel, dtype=pdt, device=dev))

        # Block-quantised gather: codes and scales as every rank would send
        # them; the other ranks' come from quantising their synthetic 16-bit
        # shards once.
        self.codes = self.scales = None
        if w.gather_bits != 16:
            cb = abi.zero_quant_code_bytes(n, w.gather_bits)
            self.codes = self._keep("codes", "gather_codes", torch.empty((w.nd, cb), dtype=torch.uint8, device=dev))
            self.scales = self._keep("scales", "gather_codes", torch.empty((w.nd, abi.zero_quant_scale_count(n)),
                                                                            dtype=torch.float32, device=dev))
            for r in range(w.nd):
                if r not in self.owners:
                    self.quantize_shard(r)

        # Per-rank pointer lists, marshalled once (the buffers never move).
        self.contrib_tables = None if w.pre_reduced else [
            abi.PointerTable(self.contribs(i), 2 * n, "contribution") for i in range(len(self.owners))]
        self.shard_table = None if self.shards is None else abi.PointerTable(list(self.shards), 2 * n, "shard")
        self.code_table = self.scale_table = None
        if self.codes is not None:
            self.code_table = abi.PointerTable(list(self.codes), self.codes.shape[1], "code shard")
            self.scale_table = abi.PointerTable(list(self.scales), 4 * self.scales.shape[1], "scale shard")

        # ZeRO-Offload: pinned staging for the chunked copies, host threads.
        self.staging = None
        self.host_threads = min(HOST_THREADS_MAX, len(os.sched_getaffinity(0)))
        if w.offload:
            chunk = min(OFFLOAD_CHUNK, max(64, n))
            self.staging = self._keep("staging", "staging_host",
                                      torch.empty(64 + 8 * chunk, dtype=torch.uint8, pin_memory=True))
        # ZeRO-Offload's one-step-delayed update: the library's persistent host
        # workers, and a device buffer for the gradient copied aside (first
        # half) and the parameters in flight (second half).
        self.offload_h = None
        if w.offload_delay:
            self.offload_h = abi.Offload(self.host_threads)
            self.offload_buffer = self._keep("offload_in_flight", "work",
                                             torch.empty(2 * n, dtype=torch.int16, device=dev))

        n_sets = 1 if w.pre_reduced else len(self.owners)
        self.ws = self._keep("workspace", "work",
                             torch.empty(abi.zero_workspace_bytes(n, n_sets), dtype=torch.uint8, device=dev))
        self.n_sets = n_sets
        self.flag = self._keep("flag", "work", torch.zeros(1, dtype=torch.int32, device=dev))
        self.norm = self._keep("norm", "work", torch.zeros(1, dtype=torch.float64, device=dev))
        self.coef = self._keep("coef", "work", torch.zeros(1, dtype=torch.float32, device=dev))

        # All owners' contributions in one launch when every rank's full local
        # gradient is a row of one block (owner o's slice at o * n).
        self.owners_table = None
        if self.local is not None and len(self.owners) > 1:
            self.owners_table = abi.PointerTable(list(self.local), 2 * self.full_numel, "contribution")

        # The device step count (a zero_step_state) and the AdamW scalars of
        # CONSTS_TABLE_LEN consecutive steps from state.table_t0.
        self.state = self._keep("step_state", "work", torch.zeros(ctypes.sizeof(abi.zero_step_state) // 8,
                                                                  dtype=torch.int64, device=dev))
        n_fields = len(abi.zero_adam_consts._fields_)
        self.consts_table = self._keep("consts_table", "work", torch.zeros((CONSTS_TABLE_LEN, n_fields),
                                                                         dtype=torch.float32, device=dev))
        self._set_step(1)
        expect = allocation_plan(w, self.plan)
        if self.ledger != expect:
            raise AssertionError(f"allocations differ from allocation_plan: {self.ledger} vs {expect}")

    def _keep(self, name, role, tensor):
        """Record an allocation (its whole storage) in the ledger; returns the tensor."""
        self.ledger.append((name, role, tensor.untyped_storage().nbytes()))
        return tensor

    # -- inputs --------------------------------------------------------------

    def _zero_padding(self, owner, t):
        """Zero the padded tail of an emulated owner's single-unit shard."""
        if self.n_units != 1:
            return
        numel, s, _, _ = self.plan.unit(0)
        real = max(0, min(numel - owner * s, s))
        t[real:].zero_()

    def fresh_gradients(self, step, tile_period=None):
        """Draw every emulated rank's full local gradient for ``step`` (padding zero)."""
        w = self.w
        psi = w.psi
        for r in range(w.nd):
            g = self.local[r]
            synth.normal_(g[:psi], w.grad_std * w.loss_scale, self.seed, 1000 * (step + 1) + r)
            synth.outliers_(g[:psi], w.outlier_frac, w.outlier_mult, self.seed, 1000 * (step + 1) + r)
            if tile_period:
                synth.tile_(g[:psi], tile_period)
            g[psi:].zero_()

    def contribs(self, i):
        """Device views of the nd contributions to emulated owner i's slice (rank order)."""
        o = self.owners[i]
        if self.local is not None:
            return [self.local[r, o * self.n:(o + 1) * self.n] for r in range(self.w.nd)]
        rank = self.w.rank
        return [self.own_grad if r == rank else self.contrib_block[r if r < rank else r - 1]
                for r in range(self.w.nd)]

    def param_out(self, i):
        o = self.owners[i]
        if self.shards is not None:
            return self.shards[o]
        if self.w.pre_reduced:
            return self.param
        return self.full[o * self.n:(o + 1) * self.n]

    def grad_of(self, i):
        return self.grad if self.w.pre_reduced else self.reduced[i]

    # -- the step count, on the device ------------------------------------------

    def hparams_at(self, t):
        w = self.w
        return abi.adam_hparams(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay, w.inv_loss_scale, t)

    def hparams(self):
        return self.hparams_at(self.t)

    def _fill_table(self, t0):
        rows = b"".join(bytes(abi.zero_adam_consts_fill(self.hparams_at(t))) for t in range(t0, t0 + CONSTS_TABLE_LEN))
        # from pageable host memory: the copy is done before this returns
        self.consts_table.copy_(torch.frombuffer(bytearray(rows), dtype=torch.float32).view_as(self.consts_table))

    def _set_step(self, t):
        """Set the device step count to t (counters cleared) and the scalars table from t."""
        torch.cuda.synchronize(self.device)
        self._fill_table(t)
        self.state.copy_(torch.frombuffer(bytearray(abi.step_state(t, t)), dtype=torch.int64))
        self._table_t0 = t
        self._step_hi = t        # the device step count is at most this

    def _ensure_table(self):
        """Before enqueueing a step: the table must hold the step's scalars.

        Each step advances the device count by at most one, so the count is at
        most _step_hi; when that may pass the table's end, wait for the device,
        read the count and refill the table from there.
        """
        if self._step_hi < self._table_t0 + CONSTS_TABLE_LEN:
            return
        torch.cuda.synchronize(self.device)
        t = int(self.state[0].item())
        self._fill_table(t)
        self.state[3] = t
        self._table_t0 = t
        self._step_hi = t

    @property
    def t(self):
        """The step count of the next update (read from the device)."""
        return int(self.state[0].item())

    @t.setter
    def t(self, value):
        self._set_step(int(value))

    def counters(self):
        """(t, applied, skipped, last_flag) from the device step state."""
        st = [int(x) for x in self.state.cpu()]
        last = st[4] & 0xFFFFFFFF               # the low half: last_flag (little-endian)
        return st[0], st[1], st[2], last - (1 << 32) if last >= 1 << 31 else last

    # -- the step ------------------------------------------------------------

    def reduce_all(self, stream=None):
        if self.owners_table is not None:
            abi.zero_reduce_owners(self.owners_table, self.n, len(self.owners), self.n, self.w.grad_dtype,
                                   self.w.inv_loss_scale, self.reduced, self.n, self.ws, self.flag, stream)
            return
        for i in range(len(self.owners)):
            abi.zero_reduce_shard(self.contrib_tables[i], self.n, self.w.grad_dtype, self.w.inv_loss_scale,
                                  self.reduced[i], self.ws, i, self.flag, stream)

    def norm_all(self, stream=None):
        w = self.w
        grad = self.grad if w.pre_reduced else None
        abi.zero_grad_norm(grad, self.n, w.grad_dtype, w.inv_loss_scale, self.ws, self.n_sets, None, 0,
                           w.max_norm, self.flag, self.norm, self.coef, stream)

    def adam_all(self, stream=None):
        w = self.w
        k = len(self.owners)
        if w.offload:
            self.flush(stream)
            hp = self.hparams()
            for i in range(k):
                abi.zero_offload_adam_step(self.master[i], self.m[i], self.v[i], self.grad_of(i), w.grad_dtype,
                                           self.n, hp, self.coef, self.flag, self.param_out(i), w.param_dtype,
                                           self.staging, self.host_threads, stream)
            return
        # Every owner in one launch: owner i's rows are i * n apart in every array
        # (the state, the reduced gradients, and the parameter buffer, where
        # owners 0..nd-1 are consecutive); one owner needs no strides.
        if k > 1:
            # all ranks emulated: owners 0..nd-1, rows of the [k, n] arrays and
            # consecutive slices of the parameter buffer (or rows of the shards)
            param = self.full if self.shards is None else self._shards_block
            grad, stride = self.reduced, self.n
        else:
            grad, param, stride = self.grad_of(0), self.param_out(0), 0
        abi.zero_adam_step_owners(self.master, self.m, self.v, stride, grad, w.grad_dtype, stride, self.n, k,
                                  self.consts_table, CONSTS_TABLE_LEN, self.state, self.coef, self.flag, param,
                                  stride, w.param_dtype, stream)

    def end_step(self, stream=None):
        abi.zero_step_end(self.flag, self.state, stream)
        self._step_hi += 1

    def quantize_shard(self, r, stream=None):
        abi.zero_quantize_blocks(self.shards[r], self.w.param_dtype, self.n, self.w.gather_bits, self.codes[r],
                                 self.scales[r], stream)

    def quantize_all(self, stream=None):
        for o in self.owners:
            self.quantize_shard(o, stream)

    def gather_unit(self, u, stream=None):
        if self.codes is not None:
            abi.zero_gather_dequant(self.plan, self.code_table, self.scale_table, u, u + 1, self.w.gather_bits,
                                    self.w.param_dtype, self.full, self.ws, stream)
        else:
            abi.zero_gather_params(self.plan, self.shard_table, u, u + 1, self.w.param_dtype, self.full,
                                   self.ws, stream)

    def gather_all(self, stream=None):
        for u in range(self.n_units):
            self.gather_unit(u, stream)

    def delayed_adam(self, stream=None):
        """ZeRO-Offload's one-step-delayed update: the previous step's host AdamW
        ends (its 16-bit parameters reach the device), then this step's begins
        and runs on the host while the GPU goes on with the next step."""
        w = self.w
        self.flush(stream)
        self.offload_h.begin(self.master[0], self.m[0], self.v[0], self.grad_of(0), w.grad_dtype, self.n,
                             self.hparams(), self.coef, self.flag, w.param_dtype, self.offload_buffer, self.staging,
                             stream)

    def flush(self, stream=None):
        """Finish a delayed host update still in flight; True if one was applied."""
        if self.offload_h is not None and self.offload_h.in_flight:
            return self.offload_h.end(self.param_out(0), stream)
        return False

    def _enqueue(self, stream=None):
        if not self.w.pre_reduced:
            self.reduce_all(stream)
        self.norm_all(stream)
        if self.offload_h is not None:
            self.delayed_adam(stream)
        else:
            self.adam_all(stream)
        if self.codes is not None:
            self.quantize_all(stream)
        if self.shards is not None:
            self.gather_all(stream)
        self.end_step(stream)

    def step(self, stream=None):
        """Enqueue one whole step; returns without synchronising.

        The flag starts each step cleared (by the previous step's end); a set
        flag skips the update and leaves the step count where it was.
        """
        self._ensure_table()
        self._enqueue(stream)

    # -- the step as a HIP graph -----------------------------------------------

    def capture(self):
        """Capture one whole step as a HIP graph (no host work inside a step).

        AdamW reads its scalars from the device table by the device step count,
        so replays need no host refresh.
        """
        if self.w.offload:
            raise ValueError("the offloaded update runs on the host and cannot be captured")
        self._ensure_table()
        self.graph = torch.cuda.CUDAGraph()
        hi = self._step_hi
        with torch.cuda.graph(self.graph):
            self._enqueue()
        self._step_hi = hi       # capturing ran nothing

    def replay(self):
        """Launch the captured step; returns without synchronising."""
        self._ensure_table()
        self.graph.replay()
        self._step_hi += 1

    # -- accounting ------------------------------------------------------------

    def phases(self):
        return phase_model(self.w, self.plan)

    def algorithmic_bytes(self):
        return sum(p["launches"] * p["bytes_per_launch"] for p in self.phases().values())


def phase_model(w, plan):
    """Kernel, launches per step and algorithmic bytes per launch of each phase.

    Algorithmic bytes are what the method must move, not counting re-reads.
    Per owned element: the reduce reads 2*Nd bytes of contributions and
    writes the 2-byte reduced gradient; AdamW reads it (2), reads and writes
    master, m and v (24) and writes the 16-bit parameter (2).  A gradient that
    arrives reduced is read once more by the norm pass (2).  A ZeRO-3 gather
    reads and writes 2 bytes per gathered element.  A block-quantised gather
    instead reads the 16-bit shard and writes its codes and scales once per
    owned element (2 + b/8 + 4/256), then reads codes and scales and writes 16
    bits per gathered element (b/8 + 4/256 + 2).  Needs no GPU.
    """
    n, _ = plan.rank(0)
    n_units = plan.info()["n_units"]
    owners = w.nd if w.all_ranks else 1
    # every owner in one launch when all ranks' local gradients are rows of one block
    reduce_launches = 1 if w.all_ranks and n_units == 1 else owners
    out = {}
    if not w.pre_reduced:
        out["reduce"] = {"kernel": "reduce_kernel", "launches": reduce_launches,
                         "bytes_per_launch": (2 * w.nd + 2) * n * owners / reduce_launches}
    out["norm"] = {"kernel": "sumsq_kernel" if w.pre_reduced else "finalize_kernel", "launches": 1,
                   "bytes_per_launch": 2 * n if w.pre_reduced else 0}
    if w.offload:
        # host memory traffic of the host AdamW (the same 28 bytes per element);
        # the 4 bytes per element over PCIe are reported separately
        out["adam"] = {"kernel": "host_adam", "launches": owners, "bytes_per_launch": 28 * n}
    else:
        out["adam"] = {"kernel": "adam_kernel", "launches": 1, "bytes_per_launch": 28 * n * owners}
    if w.gather_bits != 16:
        code = abi.zero_quant_code_bytes(n, w.gather_bits) + 4 * abi.zero_quant_scale_count(n)
        # shards are 16-byte aligned, so the span kernel runs
        out["quantize"] = {"kernel": "quantize_span_kernel", "launches": owners, "bytes_per_launch": 2 * n + code}
        out["gather"] = {"kernel": "gather_dequant_kernel", "launches": n_units,
                         "bytes_per_launch": (code + 2 * n) * w.nd / n_units}
    elif w.gather_per_unit:
        out["gather"] = {"kernel": "gather_kernel", "launches": n_units, "bytes_per_launch": 4 * n * w.nd / n_units}
    return out


def allocation_plan(w, plan):
    """Every allocation RankStep makes for workload ``w``: (buffer, role, bytes), in order.

    Roles, for the emulated rank: "params16" its 16-bit parameters, "grads16"
    its 16-bit gradients, "state32" (or "state32_host" under ZeRO-Offload) its
    fp32 master, m and v; "peers" buffers standing in for the other ranks'
    (their gradient contributions to this rank's slice, their 16-bit shards);
    "gathered" the full 16-bit parameters a ZeRO-3 rank assembles layer by
    layer for compute; "gather_codes" the quantised gather's codes and scales;
    "work" workspace, flag, norm, clip multiplier, step state and scalars
    table; "staging_host" pinned staging.  Roles prefixed "all_ranks_" belong
    to every emulated rank at once.  RankStep checks its allocations against
    this list, so it can be read without a GPU.  Needs no GPU.
    """
    n, _ = plan.rank(0)
    full = plan.full_numel()
    n_units = plan.info()["n_units"]
    k = w.nd if w.all_ranks else 1
    row = -(-n // CONTRIB_ROW_ALIGN) * CONTRIB_ROW_ALIGN
    out = []
    if w.pre_reduced:
        out.append(("grad", "grads16", 2 * n))
    elif w.all_ranks and n_units == 1:
        out += [("local", "all_ranks_grads16", 2 * w.nd * full), ("reduced", "all_ranks_grads16", 2 * k * n)]
    else:
        if w.nd > 1:
            out.append(("peer_contributions", "peers", 2 * (w.nd - 1) * row))
        out.append(("grad_full", "grads16", 2 * full) if w.stage <= 1 else ("grad_own", "grads16", 2 * row))
    role = ("all_ranks_" if k > 1 else "") + ("state32_host" if w.offload else "state32")
    out += [(name, role, 4 * k * n) for name in ("master", "m", "v")]
    if w.gather_per_unit:
        if k > 1:
            out.append(("shards", "all_ranks_params16", 2 * w.nd * n))
        else:
            out += [("shard_own", "params16", 2 * n), ("peer_shards", "peers", 2 * (w.nd - 1) * n)]
        out.append(("gathered", "gathered", 2 * full))
    elif w.pre_reduced:
        out.append(("param", "params16", 2 * n))
    else:
        out.append(("full", "all_ranks_params16" if k > 1 else "params16", 2 * full))
    if w.gather_bits != 16:
        out += [("codes", "gather_codes", w.nd * abi.zero_quant_code_bytes(n, w.gather_bits)),
                ("scales", "gather_codes", 4 * w.nd * abi.zero_quant_scale_count(n))]
    if w.offload:
        out.append(("staging", "staging_host", 64 + 8 * min(OFFLOAD_CHUNK, max(64, n))))
    if w.offload_delay:
        out.append(("offload_in_flight", "work", 4 * n))
    n_sets = 1 if w.pre_reduced else k
    out += [("workspace", "work", abi.zero_workspace_bytes(n, n_sets)), ("flag", "work", 4), ("norm", "work", 8),
            ("coef", "work", 4), ("step_state", "work", ctypes.sizeof(abi.zero_step_state)),
            ("consts_table", "work", 4 * CONSTS_TABLE_LEN * len(abi.zero_adam_consts._fields_))]
    return out


def role_bytes(w, plan):
    """Bytes per role of allocation_plan."""
    totals = {}
    for _, role, nbytes in allocation_plan(w, plan):
        totals[role] = totals.get(role, 0) + nbytes
    return totals
