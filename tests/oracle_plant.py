"""Plant a mistake in a copy of an oracle function (CPU only).

Negative controls take an oracle function's source, replace one expression
and compile the result in the oracle module's namespace, so a test can show
that a pin (or the GPU parity bar) turns red on that mistake.  The oracle
module itself is never modified."""
import inspect
import textwrap

from oracle import dit


def planted(func, old: str, new: str, count: int = 1, module=None):
    src = textwrap.dedent(inspect.getsource(func))
    assert src.count(old) >= count, f"plant target not found: {old!r}"
    src = src.replace(old, new, count)
    ns = dict(vars(module or dit))
    exec(compile(src, f"<planted {func.__name__}>", "exec"), ns)
    return ns[func.__name__]


def planted_step(block_old: str, block_new: str, count: int = 1):
    """dit_step whose blocks run a planted dit_block."""
    blk = planted(dit.dit_block, block_old, block_new, count)
    src = textwrap.dedent(inspect.getsource(dit.dit_step))
    ns = dict(vars(dit))
    ns["dit_block"] = blk
    exec(compile(src, "<planted dit_step>", "exec"), ns)
    return ns["dit_step"]


def step_with(**overrides):
    """dit_step (and the dit_block it calls) compiled in a namespace where the
    named oracle functions are replaced, e.g. a planted attention."""
    ns = dict(vars(dit))
    ns.update(overrides)
    for fn in (dit.dit_block, dit.dit_step):
        if fn.__name__ in overrides:
            continue
        exec(compile(textwrap.dedent(inspect.getsource(fn)), f"<planted {fn.__name__}>", "exec"), ns)
    return ns["dit_step"]
