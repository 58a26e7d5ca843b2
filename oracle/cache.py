"""Oracle state model: paged base K/V store, low-rank rows, views and crop.

TEST INFRASTRUCTURE: imported only by tests, the smoke check and the
CPU-baseline leg of the benchmark.

What is modelled (readings of the pages, stated once here):
  * One shared sequence holds the base-weight K/V prefix, computed once
    (LRAgent review, Fig. 2: "T0" and the trajectory blocks are cached once
    in BaseShared/BaseLRShared; paperlayer summary Sec. 2: prefix KV computed
    with adapters disabled). Agent i sees SHARED[0:b_i] followed by its own
    suffix OWN_i[0:S_i].
  * The low-rank (LR) cache holds one rank-r row X_j A per position and per
    plane. BaseShared keeps one plane per agent (A_i); BaseLRShared keeps a
    single plane computed with the shared A (LRAgent review, Fig. 3a/3b).
    An adapter-off position holds a zero row (paperlayer Sec. 2; RoleKV
    "What it does": nothing before the role header runs the adapter).
  * K carries no adapter term (LRAgent review, Fig. 7: keys are shared).
  * Storage is paged so that shared pages are physically shared (paperlayer
    Sec. 3.2 names a paged cache as the route to physical sharing). The
    pages say nothing about the allocator; the reading taken is: pages of
    ``page_size`` rows per layer, a new page always takes the lowest free id,
    and a crop frees the pages lying wholly beyond the new length.
  * Crop sets a view length for all layers; it implements the role handoff
    (RoleKV "How we built it": crop and recompute at a handoff) and the
    takeover boundary (paperlayer Sec. 2, Fig. 1-2).

Values are kept in float64: K and V rows are the exact bf16 inputs widened,
and an LR row is X_j A evaluated in float64 and never rounded.
"""
from __future__ import annotations

import numpy as np

SHARED = -1
BASE_SHARED = 0
BASE_LR_SHARED = 1
MAX_AGENTS = 16


class OracleError(Exception):
    def __init__(self, code: str, msg: str = ""):
        super().__init__(f"{code}: {msg}")
        self.code = code


def _ceil_div(a, b):
    return -(-a // b)


class _Rows:
    """Growable float64 row store with truncation."""

    def __init__(self, row_shape):
        self.row_shape = tuple(row_shape)
        self.buf = np.zeros((0,) + self.row_shape)
        self.n = 0

    def put(self, start, rows):
        rows = np.asarray(rows, dtype=np.float64)
        end = start + rows.shape[0]
        if end > self.buf.shape[0]:
            cap = max(end, 2 * self.buf.shape[0], 64)
            nb = np.zeros((cap,) + self.row_shape)
            nb[: self.n] = self.buf[: self.n]
            self.buf = nb
        self.buf[start:end] = rows
        self.n = max(self.n, end)

    def truncate(self, n):
        self.n = min(self.n, n)

    def get(self, n):
        assert n <= self.n, (n, self.n)
        return self.buf[:n]


class CacheModel:
    """Independent model of the store: lengths, page tables, rows."""

    def __init__(self, n_layers, n_q_heads, n_kv_heads, head_dim, hidden, rank,
                 n_agents, mode, page_size=64, max_pages=1024):
        ok = (n_layers >= 1 and n_kv_heads >= 1 and n_q_heads >= n_kv_heads
              and n_q_heads % n_kv_heads == 0 and head_dim in (64, 128)
              and rank in (4, 8, 16, 32) and 1 <= n_agents <= MAX_AGENTS
              and mode in (BASE_SHARED, BASE_LR_SHARED) and hidden >= 64 and hidden % 64 == 0
              and page_size >= 4 and page_size <= 1024 and (page_size & (page_size - 1)) == 0
              and max_pages >= 1)
        if not ok:
            raise OracleError("ARG", "bad config")
        self.L, self.Hq, self.Hkv, self.d = n_layers, n_q_heads, n_kv_heads, head_dim
        self.hidden, self.r, self.N, self.mode = hidden, rank, n_agents, mode
        self.ps, self.max_pages = page_size, max_pages
        self.G = n_q_heads // n_kv_heads
        self.planes = n_agents if mode == BASE_SHARED else 1
        seqs = [SHARED] + list(range(n_agents))
        self.free = [set(range(max_pages)) for _ in range(n_layers)]
        self.tables = [{s: [] for s in seqs} for _ in range(n_layers)]
        self.length = [{s: 0 for s in seqs} for _ in range(n_layers)]
        self.base_len = [0] * n_agents
        # view position from which each agent's adapter term is on (RoleKV,
        # "What it does": an activated adapter switches on after the role's
        # header; the positions before it use the base weights only)
        self.lr_begin = [0] * n_agents
        self.k = [{s: _Rows((n_kv_heads, head_dim)) for s in seqs} for _ in range(n_layers)]
        self.v = [{s: _Rows((n_kv_heads, head_dim)) for s in seqs} for _ in range(n_layers)]
        # lr[l][seq][plane]; an agent's own rows live in its own plane only
        self.lr = [{s: {p: _Rows((rank,)) for p in self._planes_of(s)} for s in seqs}
                   for _ in range(n_layers)]
        self.lr_cov = [{s: {p: 0 for p in self._planes_of(s)} for s in seqs}
                       for _ in range(n_layers)]
        self.counters = dict(base_rows_shared=0, base_rows_own=0, lr_rows=0, lr_zero_rows=0,
                             rows_cropped=0, pages_alloc=0, pages_freed=0)

    # -- helpers --------------------------------------------------------------
    def plane_of(self, agent):
        return agent if self.mode == BASE_SHARED else 0

    def _planes_of(self, seq):
        if seq == SHARED:
            return list(range(self.planes))
        return [self.plane_of(seq)]

    def _check_layer(self, layer):
        if not (0 <= layer < self.L):
            raise OracleError("ARG", "layer")

    def _check_seq(self, seq):
        if not (seq == SHARED or 0 <= seq < self.N):
            raise OracleError("ARG", "seq")

    def _free_beyond(self, layer, seq, new_len):
        keep = _ceil_div(new_len, self.ps)
        tbl = self.tables[layer][seq]
        for p in tbl[keep:]:
            self.free[layer].add(p)
            self.counters["pages_freed"] += 1
        del tbl[keep:]

    # -- operations -----------------------------------------------------------
    def append_base(self, layer, seq, k, v):
        self._check_layer(layer)
        self._check_seq(seq)
        k = np.asarray(k, dtype=np.float64)
        v = np.asarray(v, dtype=np.float64)
        n = k.shape[0]
        if k.shape != (n, self.Hkv, self.d) or v.shape != k.shape:
            raise OracleError("ARG", "k/v shape")
        if n == 0:
            return
        cur = self.length[layer][seq]
        tbl = self.tables[layer][seq]
        need = _ceil_div(cur + n, self.ps) - len(tbl)
        if need > len(self.free[layer]):
            raise OracleError("OOM", "page pool exhausted")
        for _ in range(need):
            p = min(self.free[layer])
            self.free[layer].remove(p)
            tbl.append(p)
            self.counters["pages_alloc"] += 1
        self.k[layer][seq].put(cur, k)
        self.v[layer][seq].put(cur, v)
        self.length[layer][seq] = cur + n
        self.counters["base_rows_shared" if seq == SHARED else "base_rows_own"] += n

    def append_lowrank(self, layer, seq, plane, n, x=None, a=None):
        self._check_layer(layer)
        self._check_seq(seq)
        if seq == SHARED:
            if not (0 <= plane < self.planes):
                raise OracleError("ARG", "plane")
        elif plane != self.plane_of(seq):
            raise OracleError("ARG", "plane of agent")
        if n < 0:
            raise OracleError("ARG", "n")
        if x is not None and a is None:
            raise OracleError("ARG", "A missing")
        if n == 0:
            return
        cov = self.lr_cov[layer][seq][plane]
        if cov + n > self.length[layer][seq]:
            raise OracleError("STATE", "low-rank rows ahead of base rows")
        if x is None:
            rows = np.zeros((n, self.r))
            self.counters["lr_zero_rows"] += n
        else:
            x = np.asarray(x, dtype=np.float64)
            a = np.asarray(a, dtype=np.float64)
            if x.shape != (n, self.hidden) or a.shape != (self.hidden, self.r):
                raise OracleError("ARG", "x/A shape")
            rows = x @ a            # the rank-r intermediate X A, float64, unrounded
            self.counters["lr_rows"] += n
        self.lr[layer][seq][plane].put(cov, rows)
        self.lr_cov[layer][seq][plane] = cov + n

    def append_agents(self, layer, agents, counts, k, v, x=None, a=None):
        """Several agents' own rows in one call: same as per-agent appends in order.

        Checks, in order: arguments; an empty call is a no-op; every agent's own
        LR rows must be level with its base rows (STATE); pages (OOM).
        """
        self._check_layer(layer)
        if len(agents) != len(counts) or len(agents) > self.N:
            raise OracleError("ARG", "agents")
        if len(agents) == 0:
            return
        if x is not None and a is None:
            raise OracleError("ARG", "A missing")
        if len(set(agents)) != len(agents):
            raise OracleError("ARG", "duplicate agent")
        for ag, c in zip(agents, counts):
            if not (0 <= ag < self.N) or c < 0:
                raise OracleError("ARG", "agent/count")
        tot = int(sum(counts))
        if tot == 0:
            return
        k = np.asarray(k, dtype=np.float64)
        v = np.asarray(v, dtype=np.float64)
        if k.shape != (tot, self.Hkv, self.d) or v.shape != k.shape:
            raise OracleError("ARG", "k/v shape")
        if x is not None:
            x = np.asarray(x, dtype=np.float64)
            a = np.asarray(a, dtype=np.float64)
            ash = (self.N, self.hidden, self.r) if self.mode == BASE_SHARED else (self.hidden, self.r)
            if x.shape != (tot, self.hidden) or a.shape != ash:
                raise OracleError("ARG", "x/A shape")
        for ag in agents:
            if self.lr_cov[layer][ag][self.plane_of(ag)] != self.length[layer][ag]:
                raise OracleError("STATE", "own low-rank rows lag base rows")
        need = sum(_ceil_div(self.length[layer][ag] + c, self.ps) - len(self.tables[layer][ag])
                   for ag, c in zip(agents, counts))
        if need > len(self.free[layer]):
            raise OracleError("OOM", "page pool exhausted")
        o = 0
        for ag, c in zip(agents, counts):
            self.append_base(layer, ag, k[o:o + c], v[o:o + c])
            if x is None:
                self.append_lowrank(layer, ag, self.plane_of(ag), c, None, None)
            else:
                aa = a[ag] if self.mode == BASE_SHARED else a
                self.append_lowrank(layer, ag, self.plane_of(ag), c, x[o:o + c], aa)
            o += c

    def crop(self, seq, new_len):
        self._check_seq(seq)
        if new_len < 0:
            raise OracleError("ARG", "new_len")
        L = range(self.L)
        if seq == SHARED:
            lo = max(self.base_len) if self.N else 0
            if not (lo <= new_len <= min(self.length[l][SHARED] for l in L)):
                raise OracleError("STATE", "shared crop out of range")
            for l in L:
                self.counters["rows_cropped"] += self.length[l][SHARED] - new_len
                self.length[l][SHARED] = new_len
                self.k[l][SHARED].truncate(new_len)
                self.v[l][SHARED].truncate(new_len)
                for p in self.lr_cov[l][SHARED]:
                    self.lr_cov[l][SHARED][p] = min(self.lr_cov[l][SHARED][p], new_len)
                    self.lr[l][SHARED][p].truncate(new_len)
                self._free_beyond(l, SHARED, new_len)
            return
        b = self.base_len[seq]
        S = [self.length[l][seq] for l in L]
        p = self.plane_of(seq)
        if all(s == 0 for s in S) and new_len >= b:
            if new_len > min(self.length[l][SHARED] for l in L):
                raise OracleError("STATE", "attach beyond shared length")
            self.base_len[seq] = new_len
            return
        if new_len < b:
            own = 0
        else:
            own = new_len - b
            if own > min(S):
                raise OracleError("STATE", "crop beyond view length")
        for l in L:
            self.counters["rows_cropped"] += self.length[l][seq] - own
            self.length[l][seq] = own
            self.k[l][seq].truncate(own)
            self.v[l][seq].truncate(own)
            self.lr_cov[l][seq][p] = min(self.lr_cov[l][seq][p], own)
            self.lr[l][seq][p].truncate(own)
            self._free_beyond(l, seq, own)
        if new_len < b:
            self.base_len[seq] = new_len

    # -- queries --------------------------------------------------------------
    def validate_attend(self, layer, agents, base_len, suffix_len, n_q):
        self._check_layer(layer)
        n = len(agents)
        if not (1 <= n <= self.N) or len(set(agents)) != n:
            raise OracleError("ARG", "agents")
        if len(base_len) != n or len(suffix_len) != n or len(n_q) != n:
            raise OracleError("ARG", "lengths")
        for a, b, s, nq in zip(agents, base_len, suffix_len, n_q):
            if not (0 <= a < self.N):
                raise OracleError("ARG", "agent id")
            if b != self.base_len[a] or s != self.length[layer][a]:
                raise OracleError("STATE", "caller lengths differ from the cache")
            if b + s < 1 or not (1 <= nq <= b + s):
                raise OracleError("ARG", "query count")
            p = self.plane_of(a)
            if self.lr_cov[layer][SHARED][p] < b or self.lr_cov[layer][a][p] < s:
                raise OracleError("STATE", "low-rank rows do not cover the view")

    def set_lr_begin(self, agent, pos):
        """Adapter activation offset of one agent: view positions below pos take
        no low-rank term (RoleKV, "What it does"; "Challenges we ran into":
        offsets are passed explicitly)."""
        if not (0 <= agent < self.N) or int(pos) != pos or pos < 0:
            raise OracleError("ARG", "lr_begin")
        self.lr_begin[agent] = int(pos)

    def view(self, layer, agent):
        """Agent's view at one layer: K, V_base [L][Hkv][d] and its LR rows [L][r]."""
        b = self.base_len[agent]
        s = self.length[layer][agent]
        p = self.plane_of(agent)
        k = np.concatenate([self.k[layer][SHARED].get(b), self.k[layer][agent].get(s)])
        v = np.concatenate([self.v[layer][SHARED].get(b), self.v[layer][agent].get(s)])
        lr = np.concatenate([self.lr[layer][SHARED][p].get(b), self.lr[layer][agent][p].get(s)])
        return k, v, lr

    def pages(self, layer, seq):
        return list(self.tables[layer][seq])

    def lens(self, layer):
        return dict(P=self.length[layer][SHARED], b=list(self.base_len),
                    S=[self.length[layer][a] for a in range(self.N)],
                    lr_shared=[self.lr_cov[layer][SHARED][p] for p in range(self.planes)],
                    lr_own=[self.lr_cov[layer][a][self.plane_of(a)] for a in range(self.N)])
