"""Static check of the generated gfx950 assembly: no read of an MFMA
destination register may be reachable, along any control-flow path, with
fewer wait states than the result needs (11 for the 8-pass 32x32x16 bf16
MFMA the kernels use). A branch placed between an MFMA chain and the reads
of its accumulators once let such a read through unpadded; this check keeps
every kernel free of the pattern."""
import collections
import re

NEED = 11


def _regs(tok):
    m = re.match(r"([av])\[(\d+):(\d+)\]", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([av])(\d+)$", tok)
    if m:
        return {(m.group(1), int(m.group(2)))}
    return set()


def _analyse(lines, name):
    ins = []
    for l in lines:
        t = l.split(";")[0].strip()
        if re.match(r"^\.LBB\d+_\d+:", t):
            ins.append(("LABEL", t[:-1]))
            continue
        if not t or t.startswith("."):
            continue
        ins.append((t, None))
    jumps = collections.defaultdict(list)
    for i, (t, _) in enumerate(ins):
        m = re.match(r"s_(c)?branch\w*\s+(\.LBB\d+_\d+)", t)
        if m:
            jumps[m.group(2)].append(i)

    def preds(i):
        out = []
        if i > 0 and not re.match(r"s_branch\s", ins[i - 1][0]) and \
                not ins[i - 1][0].startswith("s_endpgm"):
            out.append(i - 1)
        if ins[i][0] == "LABEL":
            out += jumps.get(ins[i][1], [])
        return out

    def cost(t):
        if t == "LABEL":
            return 0
        m = re.match(r"s_nop\s+(\d+)", t)
        return int(m.group(1)) + 1 if m else 1

    found = []
    for i, (t, _) in enumerate(ins):
        if t == "LABEL" or t.startswith("v_mfma") or t.startswith("s_"):
            continue
        parts = re.split(r"[\s,]+", t)
        first = 1 if parts[0].startswith(("ds_write", "global_store", "buffer_store")) else 2
        srcs = set()
        for tok in parts[first:]:
            srcs |= _regs(tok)
        if not srcs:
            continue
        seen = {}
        stack = [(p, 0) for p in preds(i)]
        while stack:
            j, d = stack.pop()
            if d >= NEED or seen.get(j, 1 << 30) <= d:
                continue
            seen[j] = d
            tj = ins[j][0]
            if tj.startswith("v_mfma") and _regs(re.split(r"[\s,]+", tj)[1]) & srcs:
                found.append(f"{name}: '{t}' reads the result of '{tj[:50]}' after {d} wait states")
                continue
            stack += [(p, d + cost(tj)) for p in preds(j)]
    return found


def check_assembly(text):
    """Findings (strings) for every kernel in an assembly listing."""
    found, cur, body = [], None, []
    for l in text.split("\n"):
        m = re.match(r"^(_Z\w+):", l)
        if m:
            cur, body = m.group(1), []
        elif cur:
            body.append(l)
            if "s_endpgm" in l:
                found += _analyse(body, cur)
                cur, body = None, []
    return found
