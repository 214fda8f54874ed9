"""Plain Python model of the expert pool's slot rules (see include/moe_pool.h
and the Pulsar README's MoE expert-resolve list): touch-count admission into a
hot set of n_slots - n_transient experts, transient slots for the others,
slots used in the current epoch never overwritten, prefetch without touches.
Written from the rules, slot by slot, for the CPU tests of the C++ policy."""

FREE, RESIDENT, TRANSIENT = 0, 1, 2


class PoolModel:
    def __init__(self, n_layers, n_experts, n_slots, n_transient):
        self.E = n_experts
        self.L = n_layers
        self.cap = n_slots - n_transient
        self.state = [FREE] * n_slots
        self.key = [-1] * n_slots
        self.used = [-1] * n_slots          # epoch of last placement or hit
        self.pref = [False] * n_slots
        self.touch = {}
        self.epoch = 0
        self.st = dict(epochs=0, requests=0, hits_resident=0, hits_transient=0, admitted=0,
                       transient_loads=0, promotions=0, evictions=0, prefetch_loads=0,
                       prefetch_hits=0)

    # ---- helpers
    def keys_of(self, layer, ids):
        out = []
        if not 0 <= layer < self.L:
            return out
        for e in ids:
            if 0 <= e < self.E and layer * self.E + e not in out:
                out.append(layer * self.E + e)
        return out

    def slot_of(self, k):
        return self.key.index(k) if k in self.key else -1

    def n_res(self):
        return sum(1 for s in self.state if s == RESIDENT)

    def free_ok(self, s):
        return self.used[s] < self.epoch

    def coldest(self):
        cands = [s for s in range(len(self.state)) if self.state[s] == RESIDENT and self.free_ok(s)]
        if not cands:
            return -1
        # fewest touches, then oldest use, then lowest slot
        return min(cands, key=lambda s: (self.touch.get(self.key[s], 0), self.used[s], s))

    def first_free(self):
        return self.state.index(FREE) if FREE in self.state else -1

    def lru_transient(self):
        cands = [s for s in range(len(self.state)) if self.state[s] == TRANSIENT and self.free_ok(s)]
        return min(cands, key=lambda s: (self.used[s], s)) if cands else -1

    def put(self, s, k, state):
        if self.state[s] != FREE:
            self.st["evictions"] += 1
        self.state[s], self.key[s], self.used[s], self.pref[s] = state, k, self.epoch, False

    def place(self, k):
        if self.n_res() < self.cap:
            s = self.first_free()
            if s < 0:
                s = self.lru_transient()
            if s >= 0:
                self.put(s, k, RESIDENT)
                self.st["admitted"] += 1
                return s
        else:
            r = self.coldest()
            if r >= 0 and self.touch.get(k, 0) > self.touch.get(self.key[r], 0):
                self.put(r, k, RESIDENT)
                self.st["admitted"] += 1
                return r
        s = self.first_free()
        if s < 0:
            s = self.lru_transient()
        if s < 0:
            return -1
        self.put(s, k, TRANSIENT)
        self.st["transient_loads"] += 1
        return s

    # ---- operations
    def resolve(self, layer, ids):
        saved = (list(self.state), list(self.key), list(self.used), list(self.pref),
                 dict(self.touch), self.epoch, dict(self.st))
        self.epoch += 1
        self.st["epochs"] += 1
        keys = self.keys_of(layer, ids)
        for k in keys:
            self.touch[k] = self.touch.get(k, 0) + 1
        for k in keys:
            s = self.slot_of(k)
            if s >= 0:
                self.used[s] = self.epoch
        out = []
        for k in keys:
            self.st["requests"] += 1
            s = self.slot_of(k)
            if s >= 0:
                if self.pref[s]:
                    self.st["prefetch_hits"] += 1
                    self.pref[s] = False
                if self.state[s] == RESIDENT:
                    self.st["hits_resident"] += 1
                else:
                    self.st["hits_transient"] += 1
                    if self.n_res() < self.cap:
                        self.state[s] = RESIDENT
                        self.st["promotions"] += 1
                    else:
                        r = self.coldest()
                        if r >= 0 and self.touch[k] > self.touch.get(self.key[r], 0):
                            self.state[r], self.state[s] = TRANSIENT, RESIDENT
                            self.st["promotions"] += 1
                out.append((k, s, 0))
                continue
            t = self.place(k)
            if t < 0:
                (self.state, self.key, self.used, self.pref, self.touch, self.epoch,
                 self.st) = saved
                return None
            out.append((k, t, 1))
        return out

    def prefetch(self, layer, ids):
        out = []
        for k in self.keys_of(layer, ids):
            if self.slot_of(k) >= 0:
                continue
            t = self.place(k)
            if t < 0:
                continue
            self.pref[t] = True
            self.st["prefetch_loads"] += 1
            out.append((k, t, 1))
        return out
